// Fused exact attention forward, bf16 in/out, fp32 accumulation, gfx950.
//
// What is fused ("The Attention Bottleneck -- and How FlashAttention Fixed
// It", section "The fix: tiling and fusion, never touch HBM"; "Attention Is
// Memory-Bound, and Nobody Noticed for Five Years", the fused-path paragraphs):
// one workgroup owns a block of query rows, streams the K/V rows of its
// (batch, head) slice through LDS in tiles of BC keys, and per tile computes
// the scores, updates a running row maximum and row sum (the online softmax),
// and adds the probability-weighted values into an fp32 accumulator.  Only O
// and the log-sum-exp leave the chip; the N x N score matrix never exists.
//
// Mapping to CDNA4:
//  * WAVES waves x 32 query rows.  Each wave computes S^T = K Q^T on the
//    32x32x16 bf16 MFMA, so a lane owns one query (lane % 32) and 16 keys of
//    each 32-key block; the row max/sum are a per-lane reduction plus one
//    v_permlane32_swap between the two lane halves.
//  * The same orientation is kept for O^T = V^T P^T: the score accumulator,
//    converted to bf16, is already the B operand of the second product (no
//    data movement), and the output accumulator of a lane belongs to a single
//    query, so rescaling it is a per-lane scalar multiply.
//  * Q stays in VGPRs for the whole kernel.  K and V tiles go from HBM
//    straight into LDS (buffer_load ... lds, 16 bytes per lane, no VGPR
//    staging), double-buffered so tile j+1 lands while tile j is computed.
//    K feeds the first product with ds_read_b128; the V^T operand of the
//    second product comes from ds_read_b64_tr_b16 (LDS transpose read).
//  * K runs one tile ahead of V, so the score MFMAs of tile j+1 are
//    issued before the softmax of tile j and execute on the matrix unit while
//    the vector unit exponentiates.
//  * Lazy rescaling: the running maximum is only moved (and the accumulator
//    rescaled) when some row of the wave exceeds it by more than 2^8;
//    otherwise the stale maximum is kept.  O and the row sum share the same
//    reference maximum, so O = acc / l is unchanged; the probabilities stay
//    below 2^8, well inside fp32 and bf16 range.
//  * exp is exp2 with scale*log2(e) folded into one FMA; causal tiles above
//    the diagonal are never loaded; a causal workgroup runs a long and a short
//    query block (qb and nqb-1-qb), so all carry the same work; block ids are
//    remapped so one head's query blocks share an XCD's L2.
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace attn {
namespace fwd_bf16 {

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int N;
    int nqb;           // query blocks per slice
    float scale_log2;  // scale * log2(e)
    int paired;        // causal: each workgroup runs blocks nqb-1-i and i
    int BH;            // slices (persistent kernel)
    int groups;        // workgroup groups, one per XCD (persistent kernel)
    int per_group;     // workgroups per group (persistent kernel)
    int xcds;          // L2 domains of the device (block remap)
};

template <int D, int WAVES, int BC_>
struct Tile {
    static constexpr int BR = 32 * WAVES;   // query rows per workgroup
    static constexpr int BC = BC_;          // keys per tile
    static constexpr int NB = BC / 32;      // 32-key blocks per tile
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TILE = BC * D;     // elements per K or V tile
    static constexpr int LOADS = BC * D / 512;  // wave-loads (1 KiB) per tile
    static constexpr int LOADS_PER_WAVE = LOADS / WAVES;
    static_assert(BC % 32 == 0 && LOADS % WAVES == 0, "tile loads must split evenly over waves");
    static constexpr int LDS_ELEMS = 4 * TILE;  // K[2], V[2]
};

// LDS layout of the K and V tiles: key rows of D elements with a 16-byte XOR
// swizzle against bank conflicts.  The HBM -> LDS loads put lane l's 16 bytes
// at slot 16*l of the wave's 1 KiB block and may fetch any 16 bytes of the
// tile, so src(c) names the tile bytes that land in LDS chunk c (a row-major
// chunk, swizzled within its row); the read functions give each lane's element
// offset for an MFMA operand.  Rows of 256 B (d=128) or 128 B (d=64) alias
// onto the same banks without the swizzle.  (An "operand order" layout whose
// operand reads are contiguous per quarter-wave was measured slower: its
// HBM -> LDS fetches scatter 16-byte pieces over 32 rows per wave-load.)
template <int D>
struct Layout {
    __device__ static __forceinline__ int k_swz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
    __device__ static __forceinline__ int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
    __device__ static __forceinline__ uint32_t k_src(int c) {
        const int row = c / (D / 8), pc = c % (D / 8);
        return (uint32_t)(row * D + 8 * (pc ^ k_swz(row))) * 2u;
    }
    __device__ static __forceinline__ uint32_t v_src(int c) {
        const int row = c / (D / 8), pc = c % (D / 8);
        return (uint32_t)(row * D + 8 * (pc ^ v_swz(row))) * 2u;
    }
    // K operand (A of S^T = K Q^T) of key block blk, contraction step st:
    // lane l reads K row 32*blk + l%32, head dims 16*st + 8*(l/32) .. +7.
    __device__ static __forceinline__ int k_read(int st, int blk, int lane) {
        const int r = 32 * blk + (lane & 31);
        return r * D + 8 * ((2 * st + (lane >> 5)) ^ k_swz(r));
    }
    // Transpose read r (0, 1) of the V^T operand for key step st, head-dim
    // block t: 16-lane group g covers keys 16*st + 8*r + 4*(g/2) + 0..3 and
    // dims 32*t + 16*(g%2) + 0..15, lane i of the group 4 dims of one key.
    __device__ static __forceinline__ int v_read(int st, int t, int r, int lane) {
        const int tg = lane >> 4, ti = lane & 15;
        const int key = 16 * st + 8 * r + 4 * (tg >> 1) + (ti >> 2);
        const int dd = 32 * t + 16 * (tg & 1) + 4 * (ti & 3);
        return key * D + 8 * ((dd >> 3) ^ v_swz(key)) + (dd & 7);
    }
};

constexpr float kLazyThreshold = 8.0f;  // log2 units

template <int D, bool CAUSAL, int WAVES, int BC>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kernel(Params p) {
    using T = Tile<D, WAVES, BC>;
    using L = Layout<D>;
    constexpr int BR = T::BR, NB = T::NB;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::LDS_ELEMS];
    uint16_t *const Kbuf = smem;                // [2][TILE]
    uint16_t *const Vbuf = smem + 2 * T::TILE;  // [2][TILE]

    // Causal, paired: the workgroup runs query blocks nqb-1-item and item one
    // after the other, so every workgroup gets the same number of tiles and no
    // long block starts last.  Causal, unpaired: one block, longest first.
    const bool paired = CAUSAL && p.paired != 0;
    const int logical = xcd_remap(blockIdx.x, gridDim.x, p.xcds);
    const int per = paired ? (p.nqb + 1) / 2 : p.nqb;  // workgroups per slice
    const int bh = logical / per;
    const int item = logical - bh * per;
    const int npass = (paired && p.nqb - 1 - item != item) ? 2 : 1;
    for (int pass = 0; pass < npass; ++pass) {
        const int qb = (CAUSAL && (!paired || pass == 0)) ? p.nqb - 1 - item : item;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int l32 = lane & 31;
        const int hf = lane >> 5;
        const int N = p.N;

        const size_t slice = (size_t)bh * N * D;
        const uint32_t slice_bytes = (uint32_t)N * D * 2u;
        const auto rq = make_rsrc(p.q + slice, slice_bytes);
        const auto rk = make_rsrc(p.k + slice, slice_bytes);
        const auto rv = make_rsrc(p.v + slice, slice_bytes);
        const auto ro = make_rsrc(p.o + slice, slice_bytes);

        const int r0 = qb * BR;         // first query row of this workgroup
        const int q0 = r0 + wave * 32;  // first query row of this wave
        const int qrow = q0 + l32;      // this lane's query row

        // Q fragment (B operand of S^T = K Q^T): lane holds query qrow and head
        // dims 16*s + 8*hf .. +7 for each 16-wide step s.  Rows >= N read as zero.
        bf16x8 qf[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qrow * D + 16 * s + 8 * hf) * 2u));

        // Tiles 0 .. ntiles-1 are visited; tiles 0 .. nfull-1 need no mask for
        // any row of the workgroup.
        int ntiles = (N + BC - 1) / BC;
        int nfull = N / BC;
        if (CAUSAL) {
            ntiles = min(ntiles, (r0 + BR - 1) / BC + 1);
            nfull = min(nfull, (r0 + 1) / BC);
        }

        // ---- HBM -> LDS, 16 bytes per lane ----
        // Wave-load `ins` fills LDS chunks [64*ins, 64*ins + 64); lane l writes
        // chunk 64*ins + l.  Tiles past the end of the slice read as zero (buffer
        // bounds), so loads need no guard.
        uint32_t k_off[T::LOADS_PER_WAVE], v_off[T::LOADS_PER_WAVE];
#pragma unroll
        for (int n = 0; n < T::LOADS_PER_WAVE; ++n) {
            const int c = (wave + WAVES * n) * 64 + lane;
            k_off[n] = L::k_src(c);
            v_off[n] = L::v_src(c);
        }
        auto load_k = [&](int tile, int buf) __attribute__((always_inline)) {
            const uint32_t base = (uint32_t)(tile * BC * D) * 2u;
#pragma unroll
            for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
                buf_load16_lds(rk, base + k_off[n], Kbuf + buf * T::TILE + (wave + WAVES * n) * 512);
        };
        auto load_v = [&](int tile, int buf) __attribute__((always_inline)) {
            const uint32_t base = (uint32_t)(tile * BC * D) * 2u;
#pragma unroll
            for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
                buf_load16_lds(rv, base + v_off[n], Vbuf + buf * T::TILE + (wave + WAVES * n) * 512);
        };

        // ---- per-wave compute pieces ----
        // S^T = K_tile Q^T, one 32x32 accumulator per 32-key block.
        auto scores = [&](int buf, f32x16 (&s)[NB]) __attribute__((always_inline)) {
            const uint16_t *Ks = Kbuf + buf * T::TILE;
#pragma unroll
            for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    s[b] = mfma32(*reinterpret_cast<const bf16x8 *>(Ks + L::k_read(st, b, lane)), qf[st], s[b]);
            }
        };
        // Causal: a tile with no key <= the wave's last row is skipped by the wave.
        auto active = [&](int j) __attribute__((always_inline)) { return !CAUSAL || j * BC <= q0 + 31; };

        // V^T operand for key step st and head-dim block t from two transpose
        // reads: lane l receives head dim 32*t + l%32 at keys
        // {16*st + 4*(l/32) + 0..3} (r = 0) and {16*st + 8 + 4*(l/32) + 0..3}
        // (r = 1) -- the key order of the score accumulator's lane halves.
        auto v_operand = [&](const uint16_t *Vs, int st, int t) __attribute__((always_inline)) {
            const i16x4 lo = lds_read_tr16(Vs + L::v_read(st, t, 0, lane));
            const i16x4 hi = lds_read_tr16(Vs + L::v_read(st, t, 1, lane));
            const i16x4 w[2] = {lo, hi};
            return __builtin_bit_cast(bf16x8, w);
        };

        const float c = p.scale_log2;
        float m_run = -INFINITY;  // running reference max (log2 units) for query qrow
        float l_run = 0.f;        // running sum over this lane's half of the keys
        f32x16 acc[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

        // Online softmax of score tile j: probabilities (bf16, B operand of the
        // P*V product, pb[2b], pb[2b+1] for key block b) relative to the running
        // reference maximum; the output accumulator is rescaled when it moves.
        auto softmax = [&](int j, f32x16 (&s)[NB], bf16x8 (&pb)[2 * NB], bool masked) __attribute__((always_inline)) {
            if (masked) {  // keys past the end of the sequence and, if causal, past the query
                const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = j * BC + 32 * b + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (kk > lim) s[b][r] = -INFINITY;
                    }
                }
            }
            float mx = s[0][0];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = (b == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[b][r]);
            mx = pair_max(mx) * c;  // c > 0, so scaling commutes with max
            // The reference maximum moves only when some row of the wave exceeds
            // it by more than 2^kLazyThreshold.
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyThreshold) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = fast_exp2(m_run - m_safe);
                m_run = m_safe;
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
            }
            // The row sum adds the probabilities as rounded for P*V.
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                u32x4 w[2];
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = fast_exp2(fmaf(s[b][r], c, -m_run));
                    const float p1 = fast_exp2(fmaf(s[b][r + 1], c, -m_run));
                    w[r >> 3][(r & 7) >> 1] = pack_sum_bf16x2(p0, p1, (r & 2) ? rs1 : rs0);
                }
                pb[2 * b] = __builtin_bit_cast(bf16x8, w[0]);
                pb[2 * b + 1] = __builtin_bit_cast(bf16x8, w[1]);
            }
            l_run += rs0 + rs1;
        };
        // O^T += V_tile^T P^T.
        // The V^T operands are read two products ahead, so each transpose read
        // has two MFMAs' time to return (one read in flight left the LDS
        // latency exposed before every product).
        auto pv = [&](int buf, const bf16x8 (&pb)[2 * NB]) __attribute__((always_inline)) {
            const uint16_t *Vs = Vbuf + buf * T::TILE;
            constexpr int TB = D / 32, NOPS = (BC / 16) * TB, DEPTH = 3;
            bf16x8 vo[DEPTH];
#pragma unroll
            for (int i = 0; i < DEPTH - 1; ++i) vo[i] = v_operand(Vs, i / TB, i % TB);
#pragma unroll
            for (int i = 0; i < NOPS; ++i) {
                const int nx = i + DEPTH - 1;
                if (nx < NOPS) vo[nx % DEPTH] = v_operand(Vs, nx / TB, nx % TB);
                acc[i % TB] = mfma32(vo[i % DEPTH], pb[i / TB], acc[i % TB]);
            }
        };

        // During iteration j the LDS holds K(j+1) and V(j); K(j+2) and V(j+1)
        // are in flight, into the buffers K(j) and V(j-1) have vacated.
        load_k(0, 0);
        load_v(0, 0);
        if (ntiles > 1) load_k(1, 1);
        wait_vmem();
        __syncthreads();
        f32x16 sa[NB], sb[NB];
        if (active(0)) scores(0, sa);
        // The first step refills K buffer 0 (tile 2); every wave must have
        // finished reading tile 0 from it first.
        __syncthreads();
        // CHECKED is false for steps whose tiles j and j+1 are both below
        // nfull: every wave visits them and no key needs a mask, so the
        // main loop carries no per-tile tests; the remaining steps (the
        // diagonal of a causal block, a ragged last tile) run checked.
        auto step = [&](int j, f32x16 (&cur)[NB], f32x16 (&nxt)[NB], auto checked) __attribute__((always_inline)) {
            constexpr bool CHECKED = decltype(checked)::value;
            if (j + 2 < ntiles) load_k(j + 2, j & 1);
            if (!CHECKED || j + 1 < ntiles) {
                load_v(j + 1, (j + 1) & 1);
                if (!CHECKED || active(j + 1)) scores((j + 1) & 1, nxt);
            }
            if (!CHECKED || active(j)) {
                bf16x8 pb[2 * NB];
                softmax(j, cur, pb, CHECKED && j >= nfull);
                pv(j & 1, pb);
            }
            wait_vmem();
            __syncthreads();
        };
        int j = 0;
        for (; j + 2 < nfull; j += 2) {
            step(j, sa, sb, std::false_type{});
            step(j + 1, sb, sa, std::false_type{});
        }
        for (; j + 1 < ntiles; j += 2) {
            step(j, sa, sb, std::true_type{});
            step(j + 1, sb, sa, std::true_type{});
        }
        if (j < ntiles) step(j, sa, sb, std::true_type{});

        // Epilogue: O = acc / l, lse = ln(2) * (m + log2 l).
        const float l_tot = pair_sum(l_run);
        const float inv = 1.f / l_tot;
        if (qrow < N) {
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
                    w[1] = pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
                    buf_store8(w, ro, (uint32_t)(qrow * D + 32 * t + 8 * g + 4 * hf) * 2u);
                }
            }
            if (hf == 0 && p.lse) p.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
        }
    }
}

// Persistent form of the 8-wave K-ahead kernel: one workgroup per CU walks a
// fixed list of (slice, query block) items and, during the last key tile of
// one item, already loads the next item's Q rows (into the registers the
// finished score products no longer need) and its first K and V tiles (into
// the LDS buffers the last tile no longer reads).  The next item then starts
// computing at once instead of waiting for those loads with nothing else to
// do, and the per-workgroup launch disappears.  Each item is computed exactly
// as the non-persistent kernel computes it (same tiles, same order, same
// arithmetic), so the results are identical bit for bit.
//
// Work assignment.  The grid is groups x per_group workgroups; workgroup w
// belongs to group w % groups (the dispatcher hands workgroup w to XCD
// w % groups, so one group is one XCD and shares its L2) at position
// w / groups.  Group g owns the slices g, g + groups, ... (BH % groups == 0).
// Its items run slice by slice, item k = (slice k / nqb, block k % nqb), so
// the per_group workgroups of one round (items r * per_group ..
// + per_group - 1) read the same key tiles at about the same time.  Causal
// blocks run longest first within a slice (block nqb-1 - k % nqb), and odd
// rounds are dealt in reverse, so a workgroup that drew a long block draws a
// short one next and every workgroup carries about the same number of tiles.
// (Measured on causal 32k, Q x8: dealing the group's slices side by side,
// heaviest blocks first, was 2 % slower; not reversing odd rounds, 11 %.)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void persistent_kernel(Params p) {
    constexpr int WAVES = 8, BC = 64;
    using T = Tile<D, WAVES, BC>;
    using L = Layout<D>;
    constexpr int BR = T::BR, NB = T::NB;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::LDS_ELEMS];
    uint16_t *const Kbuf = smem;                // [2][TILE]
    uint16_t *const Vbuf = smem + 2 * T::TILE;  // [2][TILE]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases in SGPRs
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int N = p.N;
    const int grp = blockIdx.x % p.groups, pos = blockIdx.x / p.groups;
    const int nsl = p.BH / p.groups;
    const int nitems = nsl * p.nqb;
    // (slice, query block) of this workgroup's item in round r; false past the end.
    auto item_of = [&](int r, int &bh, int &qb) __attribute__((always_inline)) {
        const int k = r * p.per_group + ((CAUSAL && (r & 1)) ? p.per_group - 1 - pos : pos);
        if (k >= nitems) return false;
        const int sl = k / p.nqb;
        qb = k - sl * p.nqb;
        if (CAUSAL) qb = p.nqb - 1 - qb;
        bh = grp + sl * p.groups;
        return true;
    };

    uint32_t k_off[T::LOADS_PER_WAVE], v_off[T::LOADS_PER_WAVE];
#pragma unroll
    for (int n = 0; n < T::LOADS_PER_WAVE; ++n) {
        const int c = (wave + WAVES * n) * 64 + lane;
        k_off[n] = L::k_src(c);
        v_off[n] = L::v_src(c);
    }
    const uint32_t slice_bytes = (uint32_t)N * D * 2u;
    auto rsrc = [&](const uint16_t *base, int bh) __attribute__((always_inline)) {
        return make_rsrc(base + (size_t)bh * N * D, slice_bytes);
    };
    auto load_k = [&](__amdgpu_buffer_rsrc_t r, int tile, int buf) __attribute__((always_inline)) {
        const uint32_t base = (uint32_t)(tile * BC * D) * 2u;
#pragma unroll
        for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
            buf_load16_lds_so(r, k_off[n], base, Kbuf + buf * T::TILE + (wave + WAVES * n) * 512);
    };
    auto load_v = [&](__amdgpu_buffer_rsrc_t r, int tile, int buf) __attribute__((always_inline)) {
        const uint32_t base = (uint32_t)(tile * BC * D) * 2u;
#pragma unroll
        for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
            buf_load16_lds_so(r, v_off[n], base, Vbuf + buf * T::TILE + (wave + WAVES * n) * 512);
    };
    // Q fragment (B operand of S^T = K Q^T): lane holds query row qrow and head
    // dims 16*s + 8*hf .. +7 for each 16-wide step s.  Rows >= N read as zero.
    bf16x8 qf[D / 16];
    auto load_q = [&](__amdgpu_buffer_rsrc_t r, int qrow) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qf[s] = __builtin_bit_cast(bf16x8, buf_load16(r, (uint32_t)(qrow * D + 16 * s + 8 * hf) * 2u));
    };
    auto tiles_of = [&](int qb, int &ntiles, int &nfull) __attribute__((always_inline)) {
        const int r0 = qb * BR;
        ntiles = (N + BC - 1) / BC;
        nfull = N / BC;
        if (CAUSAL) {
            ntiles = min(ntiles, (r0 + BR - 1) / BC + 1);
            nfull = min(nfull, (r0 + 1) / BC);
        }
    };

    int round = 0, bh, qb;
    if (!item_of(0, bh, qb)) return;
    {
        int nt, nf;
        tiles_of(qb, nt, nf);
        const auto rk = rsrc(p.k, bh);
        load_q(rsrc(p.q, bh), qb * BR + wave * 32 + l32);
        load_k(rk, 0, 0);
        load_v(rsrc(p.v, bh), 0, 0);
        if (nt > 1) load_k(rk, 1, 1);
    }
    bool v0_late = false;  // the next item's V tile 0 was loaded after the last barrier
    for (;;) {
        const auto rk = rsrc(p.k, bh);
        const auto rv = rsrc(p.v, bh);
        const int r0 = qb * BR;
        const int q0 = r0 + wave * 32;
        const int qrow = q0 + l32;
        int ntiles, nfull;
        tiles_of(qb, ntiles, nfull);
        int nbh = 0, nqb = 0;
        const bool has_next = item_of(round + 1, nbh, nqb);

        // S^T = K_tile Q^T, one 32x32 accumulator per 32-key block.
        auto scores = [&](int buf, f32x16 (&s)[NB]) __attribute__((always_inline)) {
            const uint16_t *Ks = Kbuf + buf * T::TILE;
#pragma unroll
            for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    s[b] = mfma32(*reinterpret_cast<const bf16x8 *>(Ks + L::k_read(st, b, lane)), qf[st], s[b]);
            }
        };
        auto active = [&](int j) __attribute__((always_inline)) { return !CAUSAL || j * BC <= q0 + 31; };
        auto v_operand = [&](const uint16_t *Vs, int st, int t) __attribute__((always_inline)) {
            const i16x4 lo = lds_read_tr16(Vs + L::v_read(st, t, 0, lane));
            const i16x4 hi = lds_read_tr16(Vs + L::v_read(st, t, 1, lane));
            const i16x4 w[2] = {lo, hi};
            return __builtin_bit_cast(bf16x8, w);
        };

        const float c = p.scale_log2;
        float m_run = -INFINITY;
        float l_run = 0.f;
        f32x16 acc[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

        auto softmax = [&](int j, f32x16 (&s)[NB], bf16x8 (&pb)[2 * NB], bool masked) __attribute__((always_inline)) {
            if (masked) {
                // Per 32-key block (wave-uniform tests): keys all at or before
                // the wave's first query and before N need no mask; keys all
                // after its last query (or at or past N) are all removed; only
                // the block on the wave's diagonal or across N compares each
                // element.  Key of element r: k0 + 4*hf + cr, cr = 8*(r/4) + r%4,
                // removed when cr > lim - k0 - 4*hf.
                const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int k0 = j * BC + 32 * b;
                    const int last = CAUSAL ? min(q0, N - 1) : N - 1;  // last key every row of the wave sees
                    const int first_out = CAUSAL ? min(q0 + 31, N - 1) : N - 1;  // keys past it are out for every row
                    if (k0 + 31 <= last) continue;
                    if (k0 > first_out) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) s[b][r] = -INFINITY;
                        continue;
                    }
                    int rel = lim - k0 - 4 * hf;
                    asm volatile("" : "+v"(rel));
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) > rel) s[b][r] = -INFINITY;
                }
            }
            float mx = s[0][0];
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = (b == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[b][r]);
            mx = pair_max(mx) * c;
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyThreshold) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = fast_exp2(m_run - m_safe);
                m_run = m_safe;
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
            }
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                u32x4 w[2];
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = fast_exp2(fmaf(s[b][r], c, -m_run));
                    const float p1 = fast_exp2(fmaf(s[b][r + 1], c, -m_run));
                    w[r >> 3][(r & 7) >> 1] = pack_sum_bf16x2(p0, p1, (r & 2) ? rs1 : rs0);
                }
                pb[2 * b] = __builtin_bit_cast(bf16x8, w[0]);
                pb[2 * b + 1] = __builtin_bit_cast(bf16x8, w[1]);
            }
            l_run += rs0 + rs1;
        };
        auto pv = [&](int buf, const bf16x8 (&pb)[2 * NB]) __attribute__((always_inline)) {
            const uint16_t *Vs = Vbuf + buf * T::TILE;
            constexpr int TB = D / 32, NOPS = (BC / 16) * TB, DEPTH = 3;
            bf16x8 vo[DEPTH];
#pragma unroll
            for (int i = 0; i < DEPTH - 1; ++i) vo[i] = v_operand(Vs, i / TB, i % TB);
#pragma unroll
            for (int i = 0; i < NOPS; ++i) {
                const int nx = i + DEPTH - 1;
                if (nx < NOPS) vo[nx % DEPTH] = v_operand(Vs, nx / TB, nx % TB);
                acc[i % TB] = mfma32(vo[i % DEPTH], pb[i / TB], acc[i % TB]);
            }
        };

        // This item's Q, K(0), V(0) and K(1) were loaded by the previous item's
        // last step (or before the loop); the barrier there made them visible,
        // except a V(0) loaded after it.
        if (round == 0 || v0_late) {
            wait_vmem();
            __syncthreads();
        }
        f32x16 sa[NB], sb[NB];
        if (active(0)) scores(0, sa);
        // The first step refills K buffer 0 (tile 2); every wave must have
        // finished reading tile 0 from it first.
        __syncthreads();
        // During step v the LDS holds K(v+1) and V(v) (buffers (v+1) & 1 and
        // v & 1); K(v+2) and V(v+1) are in flight.  In the last step the loads
        // are the next item's: Q (the score products are done with qf), K(0)
        // and K(1) (no K buffer is read any more) and, when V(v) sits in
        // buffer 1, V(0).
        v0_late = false;
        auto step = [&](int v, f32x16 (&cur)[NB], f32x16 (&nxt)[NB], auto checked) __attribute__((always_inline)) {
            constexpr bool CHECKED = decltype(checked)::value;
            if (!CHECKED || v + 2 < ntiles) load_k(rk, v + 2, v & 1);
            if (!CHECKED || v + 1 < ntiles) {
                load_v(rv, v + 1, (v + 1) & 1);
                if (!CHECKED || active(v + 1)) scores((v + 1) & 1, nxt);
            } else if (has_next) {
                int nt, nf;
                tiles_of(nqb, nt, nf);
                const auto nrk = rsrc(p.k, nbh);
                load_q(rsrc(p.q, nbh), nqb * BR + wave * 32 + l32);
                load_k(nrk, 0, 0);
                if (nt > 1) load_k(nrk, 1, 1);
                if (v & 1) load_v(rsrc(p.v, nbh), 0, 0);
                else v0_late = true;
            }
            if (!CHECKED || active(v)) {
                bf16x8 pb[2 * NB];
                softmax(v, cur, pb, CHECKED && v >= nfull);
                pv(v & 1, pb);
            }
            wait_vmem();
            __syncthreads();
        };
        // Unchecked steps: this visit's and the next visit's tiles need no
        // mask and are visited by every wave, and the loads stay in range.
        // Steps whose tiles v and v+1 both lie below nfull need no mask and are
        // visited by every wave: they run without per-tile checks.
        int v = 0;
        for (; v + 2 < nfull; v += 2) {
            step(v, sa, sb, std::false_type{});
            step(v + 1, sb, sa, std::false_type{});
        }
        for (; v + 1 < ntiles; v += 2) {
            step(v, sa, sb, std::true_type{});
            step(v + 1, sb, sa, std::true_type{});
        }
        if (v < ntiles) step(v, sa, sb, std::true_type{});
        if (v0_late) load_v(rsrc(p.v, nbh), 0, 0);  // the next item's V(0): buffer 0 is free now

        // Epilogue: O = acc / l, lse = ln(2) * (m + log2 l).
        const float l_tot = pair_sum(l_run);
        const float inv = 1.f / l_tot;
        if (qrow < N) {
            const auto ro = make_rsrc(p.o + (size_t)bh * N * D, slice_bytes);
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv);
                    w[1] = pack_bf16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv);
                    buf_store8(w, ro, (uint32_t)(qrow * D + 32 * t + 8 * g + 4 * hf) * 2u);
                }
            }
            if (hf == 0 && p.lse) p.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
        }
        if (!has_next) break;
        ++round;
        bh = nbh;
        qb = nqb;
    }
}

// Small grids (fewer query blocks than CUs): the SW waves of a workgroup
// share one block of 32*RB query rows and split its keys, wave w taking key
// tiles w, w+SW, w+2*SW, ...  Each wave streams its tiles through its own
// double-buffered LDS slots, so the loop has no workgroup barrier.  With RB = 2
// a wave computes two 32-row blocks from every K and V operand it reads.  The
// per-wave online softmax is the one above, with one 32-key block per tile.
// At the end every wave leaves (m, l, O accumulator) per row block in LDS, and
// one wave per (row block, head-dim block) pair combines the SW partials:
//     m = max_w m_w,   l = sum_w 2^(m_w - m) l_w,   O = sum_w 2^(m_w - m) O_w / l
// (the merge of online-softmax states over disjoint key sets).
// Shapes: 4 waves x 32 rows, and (non-causal, d = 64) 8 waves x 64 rows, which
// halves the tiles each wave walks one after another and the grid.
template <int D, bool CAUSAL, int SW, int RB>
__global__ __launch_bounds__(64 * SW) void split_kernel(Params p) {
    using L = Layout<D>;
    constexpr int BC = 32;                  // keys per tile
    constexpr int TILE = BC * D;            // elements per K or V tile
    constexpr int LPT = TILE * 2 / 1024;    // 1 KiB loads per K (or V) tile
    constexpr int WREG = 4 * TILE;          // per-wave LDS elements: K[2], V[2]
    constexpr int TB = D / 32;              // head-dim blocks
    static_assert(RB * 32 * D <= 2 * TILE, "the partial accumulators must fit a wave's LDS slots");
    static_assert(RB * TB <= SW, "one merging wave per (row block, head-dim block)");
    static_assert(!CAUSAL || RB == 1, "a causal row block must see an allowed key in every visited tile");
    // SW waves x (K[2], V[2]) slots, then each wave's (m, l) per row block.
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SW * WREG + SW * RB * 128 * 2];
    float *const ml = reinterpret_cast<float *>(smem + SW * WREG);  // [SW][RB][2][64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    uint16_t *const Kw = smem + wave * WREG;  // [2][TILE]
    uint16_t *const Vw = Kw + 2 * TILE;       // [2][TILE]

    const int logical = xcd_remap(blockIdx.x, gridDim.x, p.xcds);
    const int bh = logical / p.nqb;
    int qb = logical - bh * p.nqb;
    if (CAUSAL) qb = p.nqb - 1 - qb;  // longest rows first
    const int N = p.N;
    const size_t slice = (size_t)bh * N * D;
    const uint32_t slice_bytes = (uint32_t)N * D * 2u;
    const auto rq = make_rsrc(p.q + slice, slice_bytes);
    const auto rk = make_rsrc(p.k + slice, slice_bytes);
    const auto rv = make_rsrc(p.v + slice, slice_bytes);
    const auto ro = make_rsrc(p.o + slice, slice_bytes);
    const int r0 = qb * 32 * RB;

    bf16x8 qf[RB][D / 16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qf[rb][s] = __builtin_bit_cast(
                bf16x8, buf_load16(rq, (uint32_t)((r0 + 32 * rb + l32) * D + 16 * s + 8 * hf) * 2u));

    int ntiles = (N + BC - 1) / BC;
    int nfull = N / BC;
    if (CAUSAL) {
        ntiles = min(ntiles, (r0 + 31) / BC + 1);
        nfull = min(nfull, (r0 + 1) / BC);
    }
    const int mine = ntiles > wave ? (ntiles - 1 - wave) / SW + 1 : 0;  // tiles of this wave

    uint32_t k_off[LPT], v_off[LPT];
#pragma unroll
    for (int n = 0; n < LPT; ++n) {
        k_off[n] = L::k_src(n * 64 + lane);
        v_off[n] = L::v_src(n * 64 + lane);
    }
    auto load = [&](int j, int slot) __attribute__((always_inline)) {
        const uint32_t base = (uint32_t)(j * BC * D) * 2u;
#pragma unroll
        for (int n = 0; n < LPT; ++n) load16_lds_async(rk, base + k_off[n], Kw + slot * TILE + n * 512);
#pragma unroll
        for (int n = 0; n < LPT; ++n) load16_lds_async(rv, base + v_off[n], Vw + slot * TILE + n * 512);
    };

    const float c = p.scale_log2;
    float m_run[RB], l_run[RB];
    f32x16 acc[RB][TB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        m_run[rb] = -INFINITY;
        l_run[rb] = 0.f;
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[rb][t] = f32x16{};
    }

    if (mine > 0) load(wave, 0);
    for (int i = 0; i < mine; ++i) {
        const int j = wave + SW * i;
        // Tile j has landed once at most the next tile's loads are pending.
        // The slot refilled here was last read in iteration i-1 by this wave,
        // whose reads were consumed (and so completed) before it got here.
        // (Three or four slots per wave were slower: the workgroup's LDS then
        // allows one workgroup per CU.)
        if (i + 1 < mine) {
            load(j + SW, (i + 1) & 1);
            wait_vmcnt<2 * LPT>();
        } else {
            wait_vmcnt<0>();
        }
        const uint16_t *Ks = Kw + (i & 1) * TILE;
        const uint16_t *Vs = Vw + (i & 1) * TILE;
        f32x16 sc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sc[rb] = f32x16{};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const bf16x8 kop = *reinterpret_cast<const bf16x8 *>(Ks + L::k_read(st, 0, lane));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) sc[rb] = mfma32(kop, qf[rb][st], sc[rb]);
        }
        bf16x8 pb[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (j >= nfull) {  // keys past the end of the sequence and, if causal, past the query
                const int lim = CAUSAL ? min(r0 + 32 * rb + l32, N - 1) : N - 1;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = j * BC + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (kk > lim) sc[rb][r] = -INFINITY;
                }
            }
            float mx = sc[rb][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[rb][r]);
            mx = pair_max(mx) * c;
            if (__builtin_amdgcn_ballot_w64(mx > m_run[rb] + kLazyThreshold) != 0) {
                const float m_new = fmaxf(m_run[rb], mx);
                const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = fast_exp2(m_run[rb] - m_safe);
                m_run[rb] = m_safe;
                l_run[rb] *= alpha;
#pragma unroll
                for (int t = 0; t < TB; ++t) acc[rb][t] *= alpha;
            }
            float rs0 = 0.f, rs1 = 0.f;
            u32x4 w[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(sc[rb][r], c, -m_run[rb]));
                const float p1 = fast_exp2(fmaf(sc[rb][r + 1], c, -m_run[rb]));
                w[r >> 3][(r & 7) >> 1] = pack_sum_bf16x2(p0, p1, (r & 2) ? rs1 : rs0);
            }
            pb[rb][0] = __builtin_bit_cast(bf16x8, w[0]);
            pb[rb][1] = __builtin_bit_cast(bf16x8, w[1]);
            l_run[rb] += rs0 + rs1;
        }
#pragma unroll
        for (int st = 0; st < BC / 16; ++st) {
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const i16x4 lo = lds_read_tr16(Vs + L::v_read(st, t, 0, lane));
                const i16x4 hi = lds_read_tr16(Vs + L::v_read(st, t, 1, lane));
                const i16x4 w[2] = {lo, hi};
                const bf16x8 vop = __builtin_bit_cast(bf16x8, w);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) acc[rb][t] = mfma32(vop, pb[rb][st], acc[rb][t]);
            }
        }
    }

    // Partials: acc[rb][t] as 16 floats per lane in this wave's own (now idle)
    // slots, (m, l) per row block in the table after the slots.
    float *const part = reinterpret_cast<float *>(Kw);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            f32x4 *dst = reinterpret_cast<f32x4 *>(part + ((rb * TB + t) * 64 + lane) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[e] = f32x4{acc[rb][t][4 * e], acc[rb][t][4 * e + 1], acc[rb][t][4 * e + 2], acc[rb][t][4 * e + 3]};
        }
        // A wave that saw no allowed key of this row (all its tiles masked for
        // it) holds a placeholder reference; -inf keeps it out of the combined
        // maximum.  The test uses the row total so both lane halves agree.
        ml[((wave * RB + rb) * 2) * 64 + lane] = pair_sum(l_run[rb]) > 0.f ? m_run[rb] : -INFINITY;
        ml[((wave * RB + rb) * 2 + 1) * 64 + lane] = l_run[rb];
    }
    __syncthreads();

    if (wave < RB * TB) {
        const int rb = wave / TB, t = wave - rb * TB;
        const int qrow = r0 + 32 * rb + l32;
        float mw[SW], m = -INFINITY;
#pragma unroll
        for (int w = 0; w < SW; ++w) {
            mw[w] = ml[((w * RB + rb) * 2) * 64 + lane];
            m = fmaxf(m, mw[w]);
        }
        float l = 0.f;
        f32x16 o = f32x16{};
#pragma unroll
        for (int w = 0; w < SW; ++w) {
            const float f = mw[w] == -INFINITY ? 0.f : fast_exp2(mw[w] - m);
            l += f * ml[((w * RB + rb) * 2 + 1) * 64 + lane];
            const f32x4 *src = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(smem + w * WREG) +
                                                               ((rb * TB + t) * 64 + lane) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f32x4 x = src[e];
                o[4 * e] += f * x[0];
                o[4 * e + 1] += f * x[1];
                o[4 * e + 2] += f * x[2];
                o[4 * e + 3] += f * x[3];
            }
        }
        const float l_tot = pair_sum(l);
        const float inv = 1.f / l_tot;
        if (qrow < N) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(o[4 * g] * inv, o[4 * g + 1] * inv);
                w[1] = pack_bf16x2(o[4 * g + 2] * inv, o[4 * g + 3] * inv);
                buf_store8(w, ro, (uint32_t)(qrow * D + 32 * t + 8 * g + 4 * hf) * 2u);
            }
            if (t == 0 && hf == 0 && p.lse) p.lse[(size_t)bh * N + qrow] = (m + __log2f(l_tot)) * kLn2;
        }
    }
}

template <int D, bool CAUSAL, int SW, int RB>
hipError_t launch_split_shape(const FwdArgs &a, hipStream_t s) {
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.N = a.N;
    p.nqb = (a.N + 32 * RB - 1) / (32 * RB);
    p.scale_log2 = a.scale * kLog2e;
    p.paired = 0;
    p.xcds = device_shape().xcds;
    const unsigned blocks = (unsigned)a.BH * (unsigned)p.nqb;
    hipLaunchKernelGGL((split_kernel<D, CAUSAL, SW, RB>), dim3(blocks), dim3(64 * SW), 0, s, p);
    return hipGetLastError();
}

// Non-causal d = 64: 8 waves x 64 rows when the 4-wave grid would exceed one
// workgroup per CU, or when each of its waves would walk 16 or more tiles in
// turn (measured: 1x12x1024 -9 %, 1x3x2048 -6 %, 1x1x4096 -14 %; grids of
// up to one workgroup per CU with shorter walks were 15-68 % slower).
template <int D, bool CAUSAL>
hipError_t launch_split(const FwdArgs &a, hipStream_t s) {
    if constexpr (D == 64 && !CAUSAL) {
        const long long grid4 = (long long)a.BH * ((a.N + 31) / 32);
        const int walk4 = ((a.N + 31) / 32 + 3) / 4;
        if (grid4 > 256 || walk4 >= 16) return launch_split_shape<64, false, 8, 2>(a, s);
    }
    return launch_split_shape<D, CAUSAL, 4, 1>(a, s);
}

// The persistent 8-wave kernel: one workgroup per CU, grouped by XCD.  Used
// when the slices split evenly over the XCDs; false otherwise (the caller then
// launches the non-persistent kernel).
template <int D, bool CAUSAL>
bool launch_persistent(const FwdArgs &a, hipStream_t s, hipError_t &err) {
    const DeviceShape shape = device_shape();
    const int groups = shape.xcds;
    if (a.BH % groups != 0) return false;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.N = a.N;
    p.nqb = (a.N + 255) / 256;
    p.scale_log2 = a.scale * kLog2e;
    p.paired = 0;
    p.BH = a.BH;
    p.groups = groups;
    p.xcds = groups;
    const long long items_per_group = (long long)(a.BH / groups) * p.nqb;
    p.per_group = (int)std::min<long long>(shape.cus / groups, items_per_group);
    const unsigned blocks = (unsigned)(groups * p.per_group);
    hipLaunchKernelGGL((persistent_kernel<D, CAUSAL>), dim3(blocks), dim3(512), 0, s, p);
    err = hipGetLastError();
    return true;
}

template <int D, bool CAUSAL, int WAVES, int BC>
hipError_t launch(const FwdArgs &a, hipStream_t s) {
    using T = Tile<D, WAVES, BC>;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.N = a.N;
    p.nqb = (a.N + T::BR - 1) / T::BR;
    p.scale_log2 = a.scale * kLog2e;
    p.paired = CAUSAL && pair_causal_blocks((long long)a.BH * p.nqb, WAVES == 8 ? 1 : 2);
    p.xcds = device_shape().xcds;
    const unsigned blocks = (unsigned)a.BH * (unsigned)(p.paired ? (p.nqb + 1) / 2 : p.nqb);
    hipLaunchKernelGGL((kernel<D, CAUSAL, WAVES, BC>), dim3(blocks), dim3(T::THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace fwd_bf16

#ifndef ATTN_FWD_BF16_NO_DEFAULT_LAUNCHER
// 8 waves (256 query rows) per workgroup share each K/V tile and run the
// K-ahead pipeline.  4 waves (128 rows, two workgroups per CU, also K-ahead:
// 2-14 % faster than the plain loop on these shapes, bit for bit the same)
// are used when there would be fewer than 192 8-wave workgroups (three
// quarters of one per CU: at 128 the 8-wave grid leaves half the CUs idle and
// measured 11-13 % slower, at 192 and above it measured up to 15 % faster);
// for causal sequences up to 1280 keys (2048 at d = 64), where the waves of a
// 256-row block differ by up to 3.5 tiles of causal work and the shorter
// block wastes more of the whole (4 waves measured 10-11 % faster at 1280
// keys, 3 % slower at 1536 with d = 128; 3-7 % faster at 1536 and 2048 with
// d = 64); and for dense grids of one to four rounds of 8-wave workgroups
// that end in a partial round, whose last round the 8-wave grid runs with
// CUs idle while two 4-wave workgroups per CU spread it (measured 2-20 %
// faster at 1.25, 1.5, 2.5 and 3.5 rounds; 2-6 % slower at whole rounds and
// 5-6 % slower below one round).  When
// even the 4-wave grid has at most 128 workgroups (half a workgroup per CU),
// the split-key kernel runs instead: four times the workgroups, each wave a
// quarter of the keys (measured 8-37 % faster there, 40 % slower at 256).
template <int D, bool CAUSAL>
static hipError_t launch_d(const FwdArgs &a, hipStream_t s) {
    using namespace fwd_bf16;
    const long long blocks4 = (long long)a.BH * ((a.N + 127) / 128);
    if (blocks4 <= 128) return launch_split<D, CAUSAL>(a, s);
    const long long blocks8 = (long long)a.BH * ((a.N + 255) / 256);
    const long long cus = device_shape().cus;
    bool wide = blocks8 >= 192;
    if (CAUSAL) wide = wide && a.N > (D == 64 ? 2048 : 1280);
    else if (blocks8 > cus && blocks8 < 4 * cus && blocks8 % cus != 0) wide = false;
    if (!wide) return launch<D, CAUSAL, 4, 64>(a, s);
    hipError_t e;
    if (launch_fwd_bf16_persistent(a, s, e)) return e;  // instantiated in attn_fwd_bf16_persistent.hip
    if constexpr (CAUSAL) return launch<D, CAUSAL, 8, 64>(a, s);
    else return launch_fwd_bf16_dense8(a, s);  // instantiated in attn_fwd_bf16_dense.hip
}

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
    if (a.d == 128) return a.causal ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
    return a.causal ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
}
#endif

}  // namespace attn
