// Unfused ("standard") attention forward: the comparison path.
//
// This is the textbook sequence traced on "Attention Is Memory-Bound, and
// Nobody Noticed for Five Years" (read Q and K, write the N x N scores; read
// them back, softmax, write the probabilities; read those and V, write O) and
// listed in the grasp.study lesson on standard self-attention, section "The
// Computational Steps of Standard Self-Attention".  Three launches:
//   1. scores  : S = Q K^T written to the workspace (bf16 or fp32)
//   2. softmax : per row, scale, mask, subtract the max, exponentiate and
//                normalise; P overwrites S in place; lse per row
//   3. output  : O = P V
// Scale and mask sit inside the softmax launch, so the N x N matrix crosses
// device memory four times (two writes, two reads), as the pages count it.
// The kernels are written to stream that matrix efficiently (MFMA products,
// 16-byte coalesced row accesses); the point of the path is its traffic.
#include "common.h"
#include "launch.h"
#define ATTN_FWD_BF16_NO_DEFAULT_LAUNCHER
#include "attn_fwd_bf16.hip"  // LDS layout of V tiles (Layout<D>)

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// 1. Scores, bf16: S[bh, i, j] = sum_c Q[bh, i, c] K[bh, j, c]  (fp32 accumulate,
//    rounded to bf16).  A workgroup takes 128 queries (4 waves x 32) and
//    SCORES_KPW consecutive 128-key blocks; same S^T = K Q^T MFMA orientation
//    as the fused kernel.
// ---------------------------------------------------------------------------
// Key blocks per workgroup: Q stays in registers across them, and each
// block's stores drain while the next block's K tile loads and multiplies
// (dense 8k: 1 block 31.4-32.0 ms for the whole unfused path, 8 blocks
// 29.5-29.8, 16 30.0, 64 32.4).
constexpr int SCORES_KPW = 8;
template <int D, bool VEC>
__global__ __launch_bounds__(256) void scores_bf16_kernel(const uint16_t *__restrict__ Q,
                                                          const uint16_t *__restrict__ K,
                                                          uint16_t *__restrict__ S, int N, int nqb,
                                                          int nkb, int xcds) {
    constexpr int KSTR = D + 8;
    constexpr int SSTR = 128 + 8;
    constexpr int LDS_ELEMS = (128 * KSTR > 128 * SSTR) ? 128 * KSTR : 128 * SSTR;
    __shared__ __attribute__((aligned(16))) uint16_t smem[LDS_ELEMS];

    const int nkg = (nkb + SCORES_KPW - 1) / SCORES_KPW;  // key-block groups per query block
    const int logical = xcd_remap(blockIdx.x, gridDim.x, xcds);
    const int kg = logical % nkg;
    const int rest = logical / nkg;
    const int qb = rest % nqb;
    const int bh = rest / nqb;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const size_t slice = (size_t)bh * N * D;
    const uint32_t slice_bytes = (uint32_t)N * D * 2u;
    const auto rq = make_rsrc(Q + slice, slice_bytes);
    const auto rk = make_rsrc(K + slice, slice_bytes);

    const int qrow = qb * 128 + wave * 32 + l32;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)(qrow * D + 16 * s + 8 * hf) * 2u));

    for (int kk = 0; kk < SCORES_KPW; ++kk) {
        const int kb = kg * SCORES_KPW + kk;
        if (kb >= nkb) break;
        const int key0 = kb * 128;
        if (kk > 0) __syncthreads();  // the previous tile's staged rows have been read
        for (int c = tid; c < 128 * D / 8; c += 256) {
            const int row = c / (D / 8), col8 = c % (D / 8);
            *reinterpret_cast<u32x4 *>(smem + row * KSTR + col8 * 8) =
                buf_load16(rk, (uint32_t)((key0 + row) * D + col8 * 8) * 2u);
        }
        __syncthreads();

        f32x16 acc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(smem + (32 * b + l32) * KSTR + 16 * s + 8 * hf);
                acc[b] = mfma32(a, qf[s], acc[b]);
            }
        }
        __syncthreads();  // K tile no longer needed; reuse LDS to stage the output rows
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(acc[b][4 * g], acc[b][4 * g + 1]);
                w[1] = pack_bf16x2(acc[b][4 * g + 2], acc[b][4 * g + 3]);
                *reinterpret_cast<u32x2 *>(smem + (wave * 32 + l32) * SSTR + 32 * b + 8 * g + 4 * hf) = w;
            }
        }
        __syncthreads();
        for (int c = tid; c < 128 * 16; c += 256) {
            const int row = c >> 4, col = (c & 15) * 8;
            const int i = qb * 128 + row, j = key0 + col;
            if (i >= N || j >= N) continue;
            uint16_t *dst = S + ((size_t)bh * N + i) * N + j;
            const uint16_t *src = smem + row * SSTR + col;
            if (VEC) {
                // S streams through (34 GB at the dense 8k shape, far beyond L2 and
                // MALL): non-temporal stores measured 6 % faster for this kernel.
                // (The same on the softmax's in-place accesses was 8 % slower.)
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(src), reinterpret_cast<u32x4 *>(dst));
            } else {
                for (int e = 0; e < 8 && j + e < N; ++e) dst[e] = src[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 2. Row softmax, bf16, in place.  A row is held in registers (CPL 16-byte
//    chunks per lane) across WPR waves, so it is read once and written once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

template <int WPR, int CPL, bool VEC>
__global__ __launch_bounds__(256) void softmax_rows_bf16_kernel(uint16_t *__restrict__ S,
                                                                float *__restrict__ lse, int N,
                                                                long long rows, float scale_log2,
                                                                int causal) {
    constexpr int RPW = 4 / WPR;  // rows per workgroup
    constexpr int TPR = 64 * WPR; // threads per row
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long long row = (long long)blockIdx.x * RPW + wave / WPR;
    const int t = (wave % WPR) * 64 + lane;
    const bool live = row < rows;
    const int i = live ? (int)(row % N) : 0;
    const int lim = causal ? i : N - 1;  // allowed keys: j <= lim
    uint16_t *base = S + (live ? row : 0) * (long long)N;

    u32x4 x[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int j = (t + c * TPR) * 8;
        x[c] = u32x4{0u, 0u, 0u, 0u};
        if (live && j < N) {
            if (VEC) {
                x[c] = *reinterpret_cast<const u32x4 *>(base + j);
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; e < 8 && j + e < N; ++e) w[e >> 1] |= (uint32_t)base[j + e] << (16 * (e & 1));
                x[c] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }
    auto val = [&](int c, int e) -> float {  // scaled score in log2 units, -inf if masked
        const int j = (t + c * TPR) * 8 + e;
        const uint32_t w = x[c][e >> 1];
        const float s = (e & 1) ? bf16_hi(w) : bf16_lo(w);
        return j <= lim ? s * scale_log2 : -INFINITY;
    };

    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, val(c, e));
    m = wave_max(m);
    if (WPR > 1) {
        if (lane == 0) red[wave] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
    }
    float l = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) l += fast_exp2(val(c, e) - m);
    l = wave_sum(l);
    if (WPR > 1) {
        if (lane == 0) red[wave] = l;
        __syncthreads();
        l = (red[0] + red[1]) + (red[2] + red[3]);
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int j = (t + c * TPR) * 8;
        if (!live || j >= N) continue;
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
            w[h] = pack_bf16x2(fast_exp2(val(c, 2 * h) - m) * inv, fast_exp2(val(c, 2 * h + 1) - m) * inv);
        if (VEC) {
            *reinterpret_cast<u32x4 *>(base + j) = u32x4{w[0], w[1], w[2], w[3]};
        } else {
            for (int e = 0; e < 8 && j + e < N; ++e) base[j + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
    if (live && t == 0 && lse) lse[row] = (m + __log2f(l)) * kLn2;
}

// Rows too long to hold in registers: two reads of the row (online max/sum,
// then the normalised write).  One workgroup per row.
template <bool VEC>
__global__ __launch_bounds__(256) void softmax_rows_bf16_stream_kernel(uint16_t *__restrict__ S,
                                                                       float *__restrict__ lse, int N,
                                                                       float scale_log2, int causal) {
    __shared__ float red_m[4], red_l[4];
    const long long row = blockIdx.x;
    const int i = (int)(row % N);
    const int lim = causal ? i : N - 1;
    uint16_t *base = S + row * (long long)N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float m = -INFINITY, l = 0.f;
    for (int j = tid; j < N; j += 256) {
        const float s = j <= lim ? bf16_lo((uint32_t)base[j]) * scale_log2 : -INFINITY;
        if (s > m) {
            l = l * fast_exp2(m - s) + 1.f;
            m = s;
        } else if (s != -INFINITY) {
            l += fast_exp2(s - m);
        }
    }
    // Combine (m, l) pairs across the workgroup.
    float mw = wave_max(m);
    float lw = wave_sum(m == -INFINITY ? 0.f : l * fast_exp2(m - mw));
    if (lane == 0) { red_m[wave] = mw; red_l[wave] = lw; }
    __syncthreads();
    const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    float L = 0.f;
    for (int w = 0; w < 4; ++w)
        if (red_m[w] != -INFINITY) L += red_l[w] * fast_exp2(red_m[w] - M);
    const float inv = 1.f / L;
    for (int j = tid; j < N; j += 256) {
        const float s = j <= lim ? bf16_lo((uint32_t)base[j]) * scale_log2 : -INFINITY;
        base[j] = (uint16_t)(pack_bf16x2(fast_exp2(s - M) * inv, 0.f) & 0xffffu);
    }
    if (tid == 0 && lse) lse[row] = (M + __log2f(L)) * kLn2;
    (void)VEC;
}

// ---------------------------------------------------------------------------
// 3. Output, bf16: O = P V.  O^T = V^T P^T on the 32x32x16 MFMA.
//
// pv_ring_kernel (N a multiple of 8): 256 query rows per workgroup; tiles of
// 64 keys of P (256 rows x 128 B) and V (64 rows of D) go from memory straight
// into LDS through a ring of three slots, so two tiles are in flight while one
// is multiplied.  P is the one N x N read of this launch, and a tile fetched
// only one ahead leaves each iteration waiting a full memory latency.
//
// The direct-to-LDS loads are load16_lds_async (inline assembly, see
// common.h): a wave waits until at most the loads of the newer tiles are
// outstanding and then meets the barrier.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(512) void pv_ring_kernel(const uint16_t *__restrict__ P, const uint16_t *__restrict__ V,
                                                      uint16_t *__restrict__ O, int N, int nqb, int xcds) {
    using VL = fwd_bf16::Layout<D>;
    constexpr int WAVES = 8, BK = 64, STAGES = 3;
    constexpr int BR = 32 * WAVES;            // query rows per workgroup
    constexpr int PT = BR * BK;               // P tile elements (32 KiB)
    constexpr int VT = BK * D;                // V tile elements
    constexpr int SLOT = PT + VT;
    constexpr int PLW = PT * 2 / 1024 / WAVES;  // 1 KiB loads per wave per tile
    constexpr int VLW = VT * 2 / 1024 / WAVES;
    constexpr int LPT = PLW + VLW;
    static_assert(PLW * WAVES * 1024 == PT * 2 && VLW * WAVES * 1024 == VT * 2, "tile loads must split evenly");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES * SLOT];

    const int logical = xcd_remap(blockIdx.x, gridDim.x, xcds);
    const int bh = logical / nqb;
    const int qb = logical - bh * nqb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int r0 = qb * BR;
    const int nrow = min(BR, N - r0);
    // P rows r0 .. r0 + nrow - 1 of this slice; reads past them return zero.
    const auto rp = make_rsrc(P + ((size_t)bh * N + r0) * (size_t)N, (uint32_t)nrow * (uint32_t)N * 2u);
    const auto rv = make_rsrc(V + (size_t)bh * N * D, (uint32_t)N * D * 2u);
    const auto ro = make_rsrc(O + (size_t)bh * N * D, (uint32_t)N * D * 2u);

    // P tile in LDS: row r (128 B = 8 chunks of 16 B), chunk pc stored at
    // position pc ^ (r & 7) so the operand reads of 32 rows spread over banks.
    // Load n of wave w fills LDS chunks 64 (w + WAVES n) .. +63.
    uint32_t p_off[PLW], v_off[VLW];
#pragma unroll
    for (int n = 0; n < PLW; ++n) {
        const int c = (wave + WAVES * n) * 64 + lane;
        const int row = c >> 3, pc = (c & 7) ^ (row & 7);
        p_off[n] = (uint32_t)(row * N + 8 * pc) * 2u;
    }
#pragma unroll
    for (int n = 0; n < VLW; ++n) v_off[n] = VL::v_src((wave + WAVES * n) * 64 + lane);
    auto load_tile = [&](int tile, int slot) __attribute__((always_inline)) {
        uint16_t *Ps = smem + slot * SLOT;
        uint16_t *Vs = Ps + PT;
        const uint32_t pbase = (uint32_t)(tile * BK) * 2u;
        const uint32_t vbase = (uint32_t)(tile * BK * D) * 2u;
#pragma unroll
        for (int n = 0; n < PLW; ++n) load16_lds_async(rp, pbase + p_off[n], Ps + (wave + WAVES * n) * 512);
#pragma unroll
        for (int n = 0; n < VLW; ++n) load16_lds_async(rv, vbase + v_off[n], Vs + (wave + WAVES * n) * 512);
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    const int ntiles = (N + BK - 1) / BK;
    const int prow = wave * 32 + l32;  // this lane's row within the block
    const int sw = prow & 7;
#pragma unroll
    for (int t = 0; t < STAGES - 1; ++t)
        if (t < ntiles) load_tile(t, t);
    for (int jt = 0; jt < ntiles; ++jt) {
        // Tile jt has landed once at most the next tile's loads are pending.
        if (jt + 1 < ntiles) wait_vmcnt<LPT>();
        else wait_vmcnt<0>();
        __syncthreads();  // tile jt visible to all; every wave is done with tile jt - 1
        if (jt + STAGES - 1 < ntiles) load_tile(jt + STAGES - 1, (jt + STAGES - 1) % STAGES);
        const uint16_t *Ps = smem + (jt % STAGES) * SLOT;
        const uint16_t *Vs = Ps + PT;
#pragma unroll
        for (int st = 0; st < BK / 16; ++st) {
            // P^T operand: keys 16 st + 4 hf + 0..3 and 16 st + 8 + 4 hf + 0..3 (the
            // key order of the V^T operand).  Keys at or past N (the ragged last
            // tile) read the next row or zero; they are cleared here.
            const int key = jt * BK + 16 * st;
            u32x2 lo = *reinterpret_cast<const u32x2 *>(Ps + prow * BK + 8 * ((2 * st) ^ sw) + 4 * hf);
            u32x2 hi = *reinterpret_cast<const u32x2 *>(Ps + prow * BK + 8 * ((2 * st + 1) ^ sw) + 4 * hf);
            if (key >= N) lo = u32x2{0u, 0u};
            if (key + 8 >= N) hi = u32x2{0u, 0u};
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            const bf16x8 pop = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
                const i16x4 a0 = lds_read_tr16(Vs + VL::v_read(st, t, 0, lane));
                const i16x4 a1 = lds_read_tr16(Vs + VL::v_read(st, t, 1, lane));
                const i16x4 av[2] = {a0, a1};
                acc[t] = mfma32(__builtin_bit_cast(bf16x8, av), pop, acc[t]);
            }
        }
    }
    const int qrow = r0 + prow;
    if (qrow < N) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(acc[t][4 * g], acc[t][4 * g + 1]);
                w[1] = pack_bf16x2(acc[t][4 * g + 2], acc[t][4 * g + 3]);
                buf_store8(w, ro, (uint32_t)(qrow * D + 32 * t + 8 * g + 4 * hf) * 2u);
            }
        }
    }
}

// pv_bf16_kernel (N not a multiple of 8, so P rows are not 16-byte aligned):
// V tiles are transposed into LDS (double-buffered), each wave gathers its own
// 32 rows of P from memory into B-operand registers.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void pv_bf16_kernel(const uint16_t *__restrict__ P, const uint16_t *__restrict__ V,
                    uint16_t *__restrict__ O, int N, int nqb, int xcds) {
    constexpr int BC = 64;
    constexpr int VSTR = BC + 8;
    constexpr int VBUF = D * VSTR;
    constexpr int VITEMS = (BC / 4) * (D / 8);
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * VBUF];

    const int logical = xcd_remap(blockIdx.x, gridDim.x, xcds);
    const int bh = logical / nqb;
    const int qb = logical - bh * nqb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const size_t slice = (size_t)bh * N * D;
    const uint32_t slice_bytes = (uint32_t)N * D * 2u;
    const auto rv = make_rsrc(V + slice, slice_bytes);
    const auto ro = make_rsrc(O + slice, slice_bytes);
    const int qrow = qb * 128 + wave * 32 + l32;
    const uint16_t *prow = P + ((size_t)bh * N + (qrow < N ? qrow : 0)) * (size_t)N;

    const bool v_loader = (VITEMS >= 256) || (tid < VITEMS);
    const int vkg = tid / (D / 8), vdg = tid % (D / 8);
    u32x4 vst[4];
    u32x4 pst[4];
    auto gload = [&](int tile) {
        const int key0 = tile * BC;
        if (v_loader) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vst[r] = buf_load16(rv, (uint32_t)((key0 + 4 * vkg + r) * D + 8 * vdg) * 2u);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int j = key0 + 16 * st + 8 * hf;
            pst[st] = u32x4{0u, 0u, 0u, 0u};
            if (qrow < N && j < N) {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; e < 8 && j + e < N; ++e) w[e >> 1] |= (uint32_t)prow[j + e] << (16 * (e & 1));
                pst[st] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    };
    auto lstore = [&](int buf) {
        if (!v_loader) return;
        uint16_t *Vt = smem + buf * VBUF;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t a0 = vst[0][w], a1 = vst[1][w], a2 = vst[2][w], a3 = vst[3][w];
            u32x2 lo, hi;
            lo[0] = (a0 & 0xffffu) | (a1 << 16);
            lo[1] = (a2 & 0xffffu) | (a3 << 16);
            hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
            hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
            *reinterpret_cast<u32x2 *>(Vt + (8 * vdg + 2 * w) * VSTR + 4 * vkg) = lo;
            *reinterpret_cast<u32x2 *>(Vt + (8 * vdg + 2 * w + 1) * VSTR + 4 * vkg) = hi;
        }
    };

    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    const int ntiles = (N + BC - 1) / BC;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int jt = 0; jt < ntiles; ++jt) {
        const int buf = jt & 1;
        bf16x8 pf[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) pf[st] = __builtin_bit_cast(bf16x8, pst[st]);
        const bool more = jt + 1 < ntiles;
        if (more) gload(jt + 1);
        const uint16_t *Vt = smem + buf * VBUF;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Vt + (32 * t + l32) * VSTR + 16 * st + 8 * hf);
                acc[t] = mfma32(a, pf[st], acc[t]);
            }
        }
        if (more) lstore(buf ^ 1);
        __syncthreads();
    }
    if (qrow < N) {
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(acc[t][4 * g], acc[t][4 * g + 1]);
                w[1] = pack_bf16x2(acc[t][4 * g + 2], acc[t][4 * g + 3]);
                buf_store8(w, ro, (uint32_t)(qrow * D + 32 * t + 8 * g + 4 * hf) * 2u);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 unfused path: plain LDS-tiled fp32 GEMM (64x64 tile, 4x4 per thread)
// and a three-pass fp32 row softmax.
// ---------------------------------------------------------------------------
// C[M x Nc] = A[M x Kd] * (TRANS_B ? B[Nc x Kd]^T : B[Kd x Nc]), per slice.
template <bool TRANS_B>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *__restrict__ A, const float *__restrict__ Bm,
                                                       float *__restrict__ C, int M, int Nc, int Kd,
                                                       long long sA, long long sB, long long sC,
                                                       int tiles_m, int tiles_n) {
    __shared__ float As[16][64 + 1];
    __shared__ float Bs[16][64 + 1];
    const int per_slice = tiles_m * tiles_n;
    const int slice = blockIdx.x / per_slice;
    const int tile = blockIdx.x - slice * per_slice;
    const int tm = tile / tiles_n, tn = tile % tiles_n;
    A += slice * sA;
    Bm += slice * sB;
    C += slice * sC;
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < Kd; k0 += 16) {
        for (int e = tid; e < 16 * 64; e += 256) {
            const int kk = e % 16, mm = e / 16;
            const int gm = tm * 64 + mm, gk = k0 + kk;
            As[kk][mm] = (gm < M && gk < Kd) ? A[(long long)gm * Kd + gk] : 0.f;
            const int gn = tn * 64 + mm;
            float b = 0.f;
            if (gn < Nc && gk < Kd) b = TRANS_B ? Bm[(long long)gn * Kd + gk] : Bm[(long long)gk * Nc + gn];
            Bs[kk][mm] = b;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = As[kk][ty * 4 + r];
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = Bs[kk][tx * 4 + r];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[r][q] = fmaf(a[r], b[q], acc[r][q]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gm = tm * 64 + ty * 4 + r;
        if (gm >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int gn = tn * 64 + tx * 4 + q;
            if (gn < Nc) C[(long long)gm * Nc + gn] = acc[r][q];
        }
    }
}

__global__ __launch_bounds__(256) void softmax_rows_f32_kernel(float *__restrict__ S, float *__restrict__ lse,
                                                               int N, float scale_log2, int causal) {
    __shared__ float red[4];
    const long long row = blockIdx.x;
    const int i = (int)(row % N);
    const int lim = causal ? i : N - 1;
    float *base = S + row * (long long)N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float m = -INFINITY;
    for (int j = tid; j <= lim; j += 256) m = fmaxf(m, base[j] * scale_log2);
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float l = 0.f;
    for (int j = tid; j <= lim; j += 256) l += exp2f(base[j] * scale_log2 - m);
    l = wave_sum(l);
    if (lane == 0) red[wave] = l;
    __syncthreads();
    l = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.f / l;
    for (int j = tid; j < N; j += 256) base[j] = j <= lim ? exp2f(base[j] * scale_log2 - m) * inv : 0.f;
    if (tid == 0 && lse) lse[row] = (m + log2f(l)) * kLn2;
}

template <int D>
hipError_t launch_bf16(const FwdArgs &a, void *ws, hipStream_t s) {
    const int N = a.N;
    const int nqb = (N + 127) / 128;
    const bool vec = (N % 8) == 0;
    const auto *q = static_cast<const uint16_t *>(a.q);
    const auto *k = static_cast<const uint16_t *>(a.k);
    const auto *v = static_cast<const uint16_t *>(a.v);
    auto *o = static_cast<uint16_t *>(a.o);
    auto *S = static_cast<uint16_t *>(ws);
    const int xcds = device_shape().xcds;
    const unsigned g1 = (unsigned)a.BH * (unsigned)nqb * (unsigned)((nqb + SCORES_KPW - 1) / SCORES_KPW);
    if (vec)
        hipLaunchKernelGGL((scores_bf16_kernel<D, true>), dim3(g1), dim3(256), 0, s, q, k, S, N, nqb, nqb, xcds);
    else
        hipLaunchKernelGGL((scores_bf16_kernel<D, false>), dim3(g1), dim3(256), 0, s, q, k, S, N, nqb, nqb, xcds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    const long long rows = (long long)a.BH * N;
    const float sl = a.scale * kLog2e;
    const int chunks = (N + 7) / 8;
    if (chunks <= 64 * 16) {  // one wave per row
        const unsigned g2 = (unsigned)((rows + 3) / 4);
        if (vec)
            hipLaunchKernelGGL((softmax_rows_bf16_kernel<1, 16, true>), dim3(g2), dim3(256), 0, s, S, a.lse, N, rows, sl, a.causal);
        else
            hipLaunchKernelGGL((softmax_rows_bf16_kernel<1, 16, false>), dim3(g2), dim3(256), 0, s, S, a.lse, N, rows, sl, a.causal);
    } else if (chunks <= 256 * 16) {  // one workgroup per row
        const unsigned g2 = (unsigned)rows;
        if (vec)
            hipLaunchKernelGGL((softmax_rows_bf16_kernel<4, 16, true>), dim3(g2), dim3(256), 0, s, S, a.lse, N, rows, sl, a.causal);
        else
            hipLaunchKernelGGL((softmax_rows_bf16_kernel<4, 16, false>), dim3(g2), dim3(256), 0, s, S, a.lse, N, rows, sl, a.causal);
    } else {
        hipLaunchKernelGGL((softmax_rows_bf16_stream_kernel<true>), dim3((unsigned)rows), dim3(256), 0, s, S, a.lse, N, sl, a.causal);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    const unsigned g3 = (unsigned)a.BH * (unsigned)nqb;
    const int nqr = (N + 255) / 256;
    if (vec)
        hipLaunchKernelGGL((pv_ring_kernel<D>), dim3((unsigned)a.BH * (unsigned)nqr), dim3(512), 0, s, S, v, o, N, nqr, xcds);
    else
        hipLaunchKernelGGL((pv_bf16_kernel<D>), dim3(g3), dim3(256), 0, s, S, v, o, N, nqb, xcds);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_unfused_bf16(const FwdArgs &a, void *ws, hipStream_t s) {
    return a.d == 128 ? launch_bf16<128>(a, ws, s) : launch_bf16<64>(a, ws, s);
}

hipError_t launch_unfused_f32(const FwdArgs &a, void *ws, hipStream_t s) {
    const int N = a.N, D = a.d;
    const auto *q = static_cast<const float *>(a.q);
    const auto *k = static_cast<const float *>(a.k);
    const auto *v = static_cast<const float *>(a.v);
    auto *o = static_cast<float *>(a.o);
    auto *S = static_cast<float *>(ws);
    const long long sQ = (long long)N * D, sS = (long long)N * N;
    const int tn1 = (N + 63) / 64;
    hipLaunchKernelGGL((gemm_f32_kernel<true>), dim3((unsigned)a.BH * (unsigned)(tn1 * tn1)), dim3(256), 0, s,
                       q, k, S, N, N, D, sQ, sQ, sS, tn1, tn1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(softmax_rows_f32_kernel, dim3((unsigned)((long long)a.BH * N)), dim3(256), 0, s, S, a.lse,
                       N, a.scale * kLog2e, a.causal);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tn3 = (D + 63) / 64;
    hipLaunchKernelGGL((gemm_f32_kernel<false>), dim3((unsigned)a.BH * (unsigned)(tn1 * tn3)), dim3(256), 0, s,
                       S, v, o, N, D, N, sS, sQ, sQ, tn1, tn3);
    return hipGetLastError();
}

}  // namespace attn
