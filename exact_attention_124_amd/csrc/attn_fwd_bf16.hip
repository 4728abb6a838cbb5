// Fused exact attention forward, bf16 in/out, fp32 accumulation, gfx950.
//
// What is fused ("The Attention Bottleneck -- and How FlashAttention Fixed
// It", section "The fix: tiling and fusion, never touch HBM"; "Attention Is
// Memory-Bound, and Nobody Noticed for Five Years", the fused-path paragraphs):
// one workgroup owns a block of 128 query rows, streams the K/V rows of its
// (batch, head) slice through LDS in tiles of 64, and per tile computes the
// scores, updates a running row maximum and row sum (the online softmax), and
// adds the probability-weighted values into an fp32 accumulator.  Only O and
// the log-sum-exp leave the chip; the N x N score matrix never exists.
//
// Mapping to CDNA4:
//  * 4 waves x 32 query rows.  Each wave computes S^T = K Q^T on the
//    32x32x16 bf16 MFMA, so a lane owns one query (lane % 32) and 16 keys of
//    each 32-key block; the row max/sum are a per-lane reduction plus one
//    v_permlane32_swap between the two lane halves.
//  * The same orientation is kept for O^T = V^T P^T: the score accumulator,
//    converted to bf16, is already the B operand of the second product (no
//    data movement), and the output accumulator of a lane belongs to a single
//    query, so the rescale by exp2(m_old - m_new) is a per-lane scalar.
//  * Q stays in VGPRs for the whole kernel; K is kept row-major in LDS; V is
//    transposed into LDS on the way in (keys contiguous per head-dim row, in
//    the key order the score accumulator uses), so every MFMA operand read is
//    one ds_read_b128.  K/V tiles are double-buffered: tile j+1 is fetched
//    into registers with 128-bit buffer loads while tile j is computed.
//  * exp is exp2 with scale*log2(e) folded into one FMA; causal tiles above
//    the diagonal are never loaded; causal query blocks run heaviest first;
//    block ids are remapped so one head's query blocks share an XCD's L2.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int N;
    int nqb;           // query blocks per slice
    float scale_log2;  // scale * log2(e)
};

template <int D>
struct Tile {
    static constexpr int BR = 128;          // query rows per workgroup
    static constexpr int BC = 64;           // keys per tile
    static constexpr int THREADS = 256;
    static constexpr int KSTR = D + 8;      // LDS row stride of K (bf16), +16 B pad
    static constexpr int VSTR = BC + 8;     // LDS row stride of V^T (bf16), +16 B pad
    static constexpr int KBUF = BC * KSTR;  // elements per K buffer
    static constexpr int VBUF = D * VSTR;   // elements per V^T buffer
    static constexpr int LDS_ELEMS = 2 * (KBUF + VBUF);
    static constexpr int KCH = BC * D / 8 / THREADS;        // 16 B K chunks per thread
    static constexpr int VITEMS = (BC / 4) * (D / 8);       // 4-key x 8-dim V items
};

// Position of key `k` (0..63) of a tile inside a V^T row.  Within every group
// of 16 keys the order is {0-3, 8-11, 4-7, 12-15}: lane half h of the score
// accumulator holds keys {4h..4h+3, 8+4h..8+4h+3} of each 16, and this order
// makes those 8 keys contiguous, so the A operand of P*V is one 16-byte read.
__device__ __forceinline__ int vt_pos(int k) {
    return (k & ~15) + 8 * ((k >> 2) & 1) + 4 * ((k >> 3) & 1) + (k & 3);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16_kernel(Params p) {
    using T = Tile<D>;
    constexpr int BR = T::BR, BC = T::BC;
    __shared__ __attribute__((aligned(16))) uint16_t smem[T::LDS_ELEMS];

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

    // Global -> register staging of one K/V tile.
    u32x4 kst[T::KCH];
    u32x4 vst[4];
    const bool v_loader = (T::VITEMS >= T::THREADS) || (tid < T::VITEMS);
    const int vkg = tid / (D / 8);  // 4-key group of this thread's V item
    const int vdg = tid % (D / 8);  // 8-dim group

    auto gload = [&](int tile) {
        const int key0 = tile * BC;
#pragma unroll
        for (int i = 0; i < T::KCH; ++i) {
            const int c = tid + i * T::THREADS;
            const int row = c / (D / 8), col8 = c % (D / 8);
            kst[i] = buf_load16(rk, (uint32_t)((key0 + row) * D + col8 * 8) * 2u);
        }
        if (v_loader) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vst[r] = buf_load16(rv, (uint32_t)((key0 + 4 * vkg + r) * D + 8 * vdg) * 2u);
        }
    };
    auto lstore = [&](int buf) {
        uint16_t *Ks = smem + buf * T::KBUF;
#pragma unroll
        for (int i = 0; i < T::KCH; ++i) {
            const int c = tid + i * T::THREADS;
            const int row = c / (D / 8), col8 = c % (D / 8);
            *reinterpret_cast<u32x4 *>(Ks + row * T::KSTR + col8 * 8) = kst[i];
        }
        if (v_loader) {
            uint16_t *Vt = smem + 2 * T::KBUF + buf * T::VBUF;
            const int pos = vt_pos(4 * vkg);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a0 = vst[0][w], a1 = vst[1][w], a2 = vst[2][w], a3 = vst[3][w];
                u32x2 lo, hi;  // head dims 2w and 2w+1, keys 4*vkg .. +3
                lo[0] = (a0 & 0xffffu) | (a1 << 16);
                lo[1] = (a2 & 0xffffu) | (a3 << 16);
                hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                *reinterpret_cast<u32x2 *>(Vt + (8 * vdg + 2 * w) * T::VSTR + pos) = lo;
                *reinterpret_cast<u32x2 *>(Vt + (8 * vdg + 2 * w + 1) * T::VSTR + pos) = hi;
            }
        }
    };

    const float c = p.scale_log2;
    float m_run = -INFINITY;  // running max of scale*log2(e)*score for query qrow
    float l_run = 0.f;        // running sum over this lane's half of the keys
    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};

    gload(0);
    lstore(0);
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const bool more = j + 1 < ntiles;
        if (more) gload(j + 1);
        const int key0 = j * BC;
        const bool active = !CAUSAL || key0 <= q0 + 31;
        if (active) {
            const uint16_t *Ks = smem + buf * T::KBUF;
            const uint16_t *Vt = smem + 2 * T::KBUF + buf * T::VBUF;

            // S^T (two 32-key blocks) = K_j Q^T.
            f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(Ks + l32 * T::KSTR + 16 * st + 8 * hf);
                const bf16x8 a1 =
                    *reinterpret_cast<const bf16x8 *>(Ks + (32 + l32) * T::KSTR + 16 * st + 8 * hf);
                s0 = mfma32(a0, qf[st], s0);
                s1 = mfma32(a1, qf[st], s1);
            }

            // Mask keys past the end of the sequence and, if causal, past the query.
            const bool need_mask = (CAUSAL && key0 + BC - 1 > q0) || (key0 + BC > N);
            if (need_mask) {
                const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = key0 + 8 * (r >> 2) + 4 * hf + (r & 3);
                    if (kk > lim) s0[r] = -INFINITY;
                    if (kk + 32 > lim) s1[r] = -INFINITY;
                }
            }

            // Online softmax update (base 2; c > 0 so max commutes with scaling).
            float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
            mx = pair_max(mx);
            const float m_new = fmaxf(m_run, mx * c);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            m_run = m_new;
#pragma unroll
            for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;

            bf16x8 pb[4];
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p0 = fast_exp2(fmaf(s0[r], c, -m_use));
                const float p1 = fast_exp2(fmaf(s1[r], c, -m_use));
                rs += p0 + p1;
                pb[r >> 3][r & 7] = (__bf16)p0;
                pb[2 + (r >> 3)][r & 7] = (__bf16)p1;
            }
            l_run = l_run * alpha + rs;

            // O^T += V_j^T P^T.
#pragma unroll
            for (int st = 0; st < 4; ++st) {
#pragma unroll
                for (int t = 0; t < D / 32; ++t) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8 *>(Vt + (32 * t + l32) * T::VSTR + 16 * st + 8 * hf);
                    acc[t] = mfma32(a, pb[st], acc[t]);
                }
            }
        }
        if (more) lstore(buf ^ 1);
        __syncthreads();
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

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t s) {
    Params p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.lse = a.lse;
    p.N = a.N;
    p.nqb = (a.N + Tile<D>::BR - 1) / Tile<D>::BR;
    p.scale_log2 = a.scale * kLog2e;
    const unsigned blocks = (unsigned)a.BH * (unsigned)p.nqb;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3(blocks), dim3(Tile<D>::THREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
    return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace attn
