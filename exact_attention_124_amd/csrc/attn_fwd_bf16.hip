// Fused exact attention forward, bf16 in/out, fp32 accumulation, gfx950.
//
// What is fused ("The Attention Bottleneck -- and How FlashAttention Fixed
// It", section "The fix: tiling and fusion, never touch HBM"; "Attention Is
// Memory-Bound, and Nobody Noticed for Five Years", the fused-path paragraphs):
// one workgroup owns a block of query rows, streams the K/V rows of its
// (batch, head) slice through LDS in tiles of 64, and per tile computes the
// scores, updates a running row maximum and row sum (the online softmax), and
// adds the probability-weighted values into an fp32 accumulator.  Only O and
// the log-sum-exp leave the chip; the N x N score matrix never exists.
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
//    staging), row-major with a 16-byte XOR swizzle against bank conflicts,
//    double-buffered so tile j+1 lands while tile j is computed.  K feeds the
//    first product with ds_read_b128; the V^T operand of the second product is
//    read from row-major V with ds_read_b64_tr_b16 (LDS transpose read).
//  * Software pipelining (PIPE): K runs one tile ahead of V, so the score
//    MFMAs of tile j+1 are issued before the softmax of tile j and execute on
//    the matrix unit while the vector unit exponentiates.
//  * Lazy rescaling (LAZY): the running maximum is only moved (and the
//    accumulator rescaled) when some row of the wave exceeds it by more than
//    2^8; otherwise the stale maximum is kept.  O and the row sum share the
//    same reference maximum, so O = acc / l is unchanged; the probabilities
//    stay below 2^8, well inside fp32 and bf16 range.
//  * exp is exp2 with scale*log2(e) folded into one FMA; causal tiles above
//    the diagonal are never loaded; causal query blocks run heaviest first;
//    block ids are remapped so one head's query blocks share an XCD's L2.
#include "common.h"
#include "launch.h"

namespace attn {
namespace fwd_bf16 {

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int N;
    int nqb;           // query blocks per slice
    float scale_log2;  // scale * log2(e)
};

template <int D, int WAVES>
struct Tile {
    static constexpr int BR = 32 * WAVES;   // query rows per workgroup
    static constexpr int BC = 64;           // keys per tile
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int CH = D / 8;        // 16-byte chunks per K/V row
    static constexpr int TILE = BC * D;     // elements per K or V tile
    static constexpr int LOADS = BC * CH / 64;          // wave-loads (1 KB) per tile
    static constexpr int LOADS_PER_WAVE = LOADS / WAVES;
    static_assert(LOADS % WAVES == 0, "tile loads must split evenly over waves");
    static constexpr int LDS_ELEMS = 4 * TILE;           // K[2], V[2]
};

// 16-byte-chunk XOR swizzles of the row-major LDS tiles.  K rows are read as
// 32 rows x one chunk per half-wave (MFMA A operand); V rows are read by the
// transpose loads as 4 rows x 4 chunks per 16 lanes.  Rows of 256 B (d=128)
// or 128 B (d=64) alias onto the same banks without a swizzle.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

constexpr float kLazyThreshold = 8.0f;  // log2 units

template <int D, bool CAUSAL, int WAVES, bool PIPE, bool LAZY>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void kernel(Params p) {
    using T = Tile<D, WAVES>;
    constexpr int BR = T::BR, BC = T::BC, CH = T::CH;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[T::LDS_ELEMS];
    uint16_t *const Kbuf = smem;                // [2][TILE]
    uint16_t *const Vbuf = smem + 2 * T::TILE;  // [2][TILE]

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nqb;
    int qb = logical - bh * p.nqb;
    if (CAUSAL) qb = p.nqb - 1 - qb;  // longest rows first

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

    const int q0 = qb * BR + wave * 32;  // first query row of this wave
    const int qrow = q0 + l32;           // this lane's query row

    // Q fragment (B operand of S^T = K Q^T): lane holds query qrow and head
    // dims 16*s + 8*hf .. +7 for each 16-wide step s.  Rows >= N read as zero.
    bf16x8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qrow * D + 16 * s + 8 * hf) * 2u));

    int ntiles = (N + BC - 1) / BC;
    if (CAUSAL) ntiles = min(ntiles, (qb * BR + BR + BC - 1) / BC);

    // ---- HBM -> LDS, 16 bytes per lane, swizzled row-major ----
    // Wave-load `ins` fills LDS chunks [64*ins, 64*ins + 64): lane l writes
    // chunk c = 64*ins + l = row * CH + physical chunk.
    uint32_t k_off[T::LOADS_PER_WAVE], v_off[T::LOADS_PER_WAVE];
#pragma unroll
    for (int n = 0; n < T::LOADS_PER_WAVE; ++n) {
        const int c = (wave + WAVES * n) * 64 + lane;
        const int row = c / CH, pc = c % CH;
        k_off[n] = (uint32_t)(row * D + 8 * (pc ^ k_swz<D>(row))) * 2u;
        v_off[n] = (uint32_t)(row * D + 8 * (pc ^ v_swz<D>(row))) * 2u;
    }
    auto load_k = [&](int tile, int buf) {
        const uint32_t base = (uint32_t)(tile * BC * D) * 2u;
#pragma unroll
        for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
            buf_load16_lds(rk, base + k_off[n], Kbuf + buf * T::TILE + (wave + WAVES * n) * 512);
    };
    auto load_v = [&](int tile, int buf) {
        const uint32_t base = (uint32_t)(tile * BC * D) * 2u;
#pragma unroll
        for (int n = 0; n < T::LOADS_PER_WAVE; ++n)
            buf_load16_lds(rv, base + v_off[n], Vbuf + buf * T::TILE + (wave + WAVES * n) * 512);
    };

    // ---- per-wave compute pieces ----
    // K operand: row (32*blk + l32), logical chunk 2*st + hf.
    auto scores = [&](int buf, f32x16 &s0, f32x16 &s1) {  // S^T = K_tile Q^T
        const uint16_t *Ks = Kbuf + buf * T::TILE;
        s0 = f32x16{};
        s1 = f32x16{};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const int r0 = l32, r1 = 32 + l32;
            const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(Ks + r0 * D + 8 * ((2 * st + hf) ^ k_swz<D>(r0)));
            const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(Ks + r1 * D + 8 * ((2 * st + hf) ^ k_swz<D>(r1)));
            s0 = mfma32(a0, qf[st], s0);
            s1 = mfma32(a1, qf[st], s1);
        }
    };
    auto tile_active = [&](int j) { return !CAUSAL || j * BC <= q0 + 31; };

    // V^T operand for key step st and head-dim block t, via two transpose
    // reads: lane (group g = lane/16, i = lane%16) addresses key
    // 16*st + 8*r + 4*(g/2) + i/4 and head dims 32*t + 16*(g%2) + 4*(i%4),
    // so lane l receives head dim 32*t + l%32 at keys
    // {16*st + 4*(l/32) + 0..3} (r = 0) and {16*st + 8 + 4*(l/32) + 0..3}
    // (r = 1): the key order of the score accumulator's lane halves.
    const int tg = lane >> 4, ti = lane & 15;
    const int v_key = 4 * (tg >> 1) + (ti >> 2);     // + 16*st + 8*r
    const int v_dim = 16 * (tg & 1) + 4 * (ti & 3);  // + 32*t
    auto v_operand = [&](const uint16_t *Vs, int st, int t) {
        const int k0 = 16 * st + v_key, k1 = k0 + 8;
        const int dd = 32 * t + v_dim;
        const uint16_t *p0 = Vs + k0 * D + 8 * ((dd >> 3) ^ v_swz<D>(k0)) + (dd & 7);
        const uint16_t *p1 = Vs + k1 * D + 8 * ((dd >> 3) ^ v_swz<D>(k1)) + (dd & 7);
        const i16x4 lo = lds_read_tr16(p0), hi = lds_read_tr16(p1);
        const i16x4 w[2] = {lo, hi};
        return __builtin_bit_cast(bf16x8, w);
    };

    const float c = p.scale_log2;
    float m_run = -INFINITY;  // running reference max (log2 units) for query qrow
    float l_run = 0.f;        // running sum over this lane's half of the keys
    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

    // Softmax of one score tile and the P*V update.
    auto consume = [&](int j, int vb, f32x16 &s0, f32x16 &s1) {
        const int key0 = j * BC;
        // Mask keys past the end of the sequence and, if causal, past the query.
        if ((CAUSAL && key0 + BC - 1 > q0) || key0 + BC > N) {
            const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = key0 + 8 * (r >> 2) + 4 * hf + (r & 3);
                if (kk > lim) s0[r] = -INFINITY;
                if (kk + 32 > lim) s1[r] = -INFINITY;
            }
        }
        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
        mx = pair_max(mx) * c;  // c > 0, so scaling commutes with max
        bool move;
        if (LAZY) move = __builtin_amdgcn_ballot_w64(mx > m_run + kLazyThreshold) != 0;
        else move = true;
        float alpha = 1.f;
        if (move) {
            const float m_new = fmaxf(m_run, mx);
            const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
            alpha = fast_exp2(m_run - m_safe);
            m_run = m_safe;
        }
        const float m_use = m_run;
        bf16x8 pb[4];
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p0 = fast_exp2(fmaf(s0[r], c, -m_use));
            const float p1 = fast_exp2(fmaf(s1[r], c, -m_use));
            rs0 += p0;
            rs1 += p1;
            pb[r >> 3][r & 7] = (__bf16)p0;
            pb[2 + (r >> 3)][r & 7] = (__bf16)p1;
        }
        if (move) {
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
        }
        l_run += rs0 + rs1;
        // O^T += V_j^T P^T.
        const uint16_t *Vs = Vbuf + vb * T::TILE;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int t = 0; t < D / 32; ++t) acc[t] = mfma32(v_operand(Vs, st, t), pb[st], acc[t]);
        }
    };

    if (PIPE) {
        // During iteration j the LDS holds K(j+1) and V(j); K(j+2) and V(j+1)
        // are in flight.
        load_k(0, 0);
        load_v(0, 0);
        if (ntiles > 1) load_k(1, 1);
        wait_vmem();
        __syncthreads();
        f32x16 sa0, sa1, sb0, sb1;
        if (tile_active(0)) scores(0, sa0, sa1);
        auto step = [&](int j, f32x16 &c0, f32x16 &c1, f32x16 &n0, f32x16 &n1) {
            if (j + 2 < ntiles) load_k(j + 2, j & 1);
            if (j + 1 < ntiles) {
                load_v(j + 1, (j + 1) & 1);
                if (tile_active(j + 1)) scores((j + 1) & 1, n0, n1);
            }
            if (tile_active(j)) consume(j, j & 1, c0, c1);
            wait_vmem();
            __syncthreads();
        };
        int j = 0;
        for (; j + 1 < ntiles; j += 2) {
            step(j, sa0, sa1, sb0, sb1);
            step(j + 1, sb0, sb1, sa0, sa1);
        }
        if (j < ntiles) step(j, sa0, sa1, sb0, sb1);
    } else {
        load_k(0, 0);
        load_v(0, 0);
        wait_vmem();
        __syncthreads();
        for (int j = 0; j < ntiles; ++j) {
            const int buf = j & 1;
            if (j + 1 < ntiles) {
                load_k(j + 1, buf ^ 1);
                load_v(j + 1, buf ^ 1);
            }
            if (tile_active(j)) {
                f32x16 s0, s1;
                scores(buf, s0, s1);
                consume(j, buf, s0, s1);
            }
            wait_vmem();
            __syncthreads();
        }
    }

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

template <int D, bool CAUSAL, int WAVES, bool PIPE, bool LAZY>
hipError_t launch(const FwdArgs &a, hipStream_t s) {
    using T = Tile<D, WAVES>;
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.N = a.N;
    p.nqb = (a.N + T::BR - 1) / T::BR;
    p.scale_log2 = a.scale * kLog2e;
    const unsigned blocks = (unsigned)a.BH * (unsigned)p.nqb;
    hipLaunchKernelGGL((kernel<D, CAUSAL, WAVES, PIPE, LAZY>), dim3(blocks), dim3(T::THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace fwd_bf16

#ifndef ATTN_FWD_BF16_NO_DEFAULT_LAUNCHER
// 8 waves (256 query rows) per workgroup share each K/V tile; when that leaves
// fewer than four workgroups per CU, 4 waves (128 rows, two workgroups per CU)
// keep the chip busier.
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
    using namespace fwd_bf16;
    const long long blocks8 = (long long)a.BH * ((a.N + 255) / 256);
    const bool wide = blocks8 >= 4 * 256;
    if (a.d == 128) {
        if (a.causal)
            return wide ? launch<128, true, 8, true, true>(a, s) : launch<128, true, 4, false, true>(a, s);
        return wide ? launch<128, false, 8, true, true>(a, s) : launch<128, false, 4, false, true>(a, s);
    }
    if (a.causal)
        return wide ? launch<64, true, 8, true, true>(a, s) : launch<64, true, 4, false, true>(a, s);
    return wide ? launch<64, false, 8, true, true>(a, s) : launch<64, false, 4, false, true>(a, s);
}
#endif

}  // namespace attn
