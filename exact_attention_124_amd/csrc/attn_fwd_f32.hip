// Fused exact attention forward in fp32 (inputs, arithmetic and output).
//
// Same fused structure as the bf16 kernel -- one workgroup per block of 128
// query rows, K/V tiles streamed through LDS, running max and running sum per
// row, only O and the log-sum-exp written ("The Attention Bottleneck -- and
// How FlashAttention Fixed It", section "The fix: tiling and fusion, never
// touch HBM") -- but on the fp32 vector units, with no reduced-precision step,
// for callers that need fp32 results.
//
// Layout: 4 waves x 32 rows; lane (l % 32) owns one query row and lane half
// (l / 32) owns half of the head dimension, for both the query and the output
// accumulator.  A score is the sum of the two halves' partial dot products
// (v_permlane32_swap).  K/V rows are read from LDS as broadcasts.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

struct Params {
    const float *q, *k, *v;
    float *o;
    float *lse;
    int N;
    int nqb;
    float scale_log2;
};

constexpr int BR = 128;  // query rows per workgroup
constexpr int BC = 32;   // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(Params p) {
    constexpr int HALF = D / 2;
    constexpr int STR = D + 4;  // LDS row stride (floats)
    __shared__ __attribute__((aligned(16))) float Ks[BC * STR];
    __shared__ __attribute__((aligned(16))) float Vs[BC * STR];

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = logical / p.nqb;
    int qb = logical - bh * p.nqb;
    if (CAUSAL) qb = p.nqb - 1 - qb;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int N = p.N;
    const size_t slice = (size_t)bh * N * D;
    const uint32_t slice_bytes = (uint32_t)N * D * 4u;
    const auto rq = make_rsrc(p.q + slice, slice_bytes);
    const auto rk = make_rsrc(p.k + slice, slice_bytes);
    const auto rv = make_rsrc(p.v + slice, slice_bytes);
    const auto ro = make_rsrc(p.o + slice, slice_bytes);

    const int q0 = qb * BR + wave * 32;
    const int qrow = q0 + l32;

    float qv[HALF];
#pragma unroll
    for (int c4 = 0; c4 < HALF / 4; ++c4) {
        const u32x4 x = buf_load16(rq, (uint32_t)(qrow * D + hf * HALF + 4 * c4) * 4u);
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[4 * c4 + e] = __uint_as_float(x[e]);
    }

    float acc[HALF];
#pragma unroll
    for (int c = 0; c < HALF; ++c) acc[c] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float cl = p.scale_log2;

    int ntiles = (N + BC - 1) / BC;
    if (CAUSAL) ntiles = min(ntiles, (qb * BR + BR + BC - 1) / BC);

    for (int j = 0; j < ntiles; ++j) {
        const int key0 = j * BC;
        __syncthreads();  // previous tile fully consumed
        // Load K and V tile (BC rows x D floats) as 16-byte chunks; rows >= N read as 0.
        for (int ch = tid; ch < BC * D / 4; ch += 256) {
            const int row = ch / (D / 4), col4 = ch % (D / 4);
            const uint32_t off = (uint32_t)((key0 + row) * D + 4 * col4) * 4u;
            *reinterpret_cast<u32x4 *>(Ks + row * STR + 4 * col4) = buf_load16(rk, off);
            *reinterpret_cast<u32x4 *>(Vs + row * STR + 4 * col4) = buf_load16(rv, off);
        }
        __syncthreads();
        if (CAUSAL && key0 > q0 + 31) continue;  // whole tile masked for this wave

        float s[BC];
#pragma unroll
        for (int kk = 0; kk < BC; ++kk) {
            const float *kr = Ks + kk * STR + hf * HALF;
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < HALF; ++c) part = fmaf(qv[c], kr[c], part);
            s[kk] = pair_sum(part);
        }
        const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;
        if ((CAUSAL && key0 + BC - 1 > q0) || key0 + BC > N) {
#pragma unroll
            for (int kk = 0; kk < BC; ++kk)
                if (key0 + kk > lim) s[kk] = -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int kk = 1; kk < BC; ++kk) mx = fmaxf(mx, s[kk]);
        const float m_new = fmaxf(m_run, mx * cl);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kk = 0; kk < BC; ++kk) {
            s[kk] = exp2f(fmaf(s[kk], cl, -m_use));
            rs += s[kk];
        }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int c = 0; c < HALF; ++c) acc[c] *= alpha;
#pragma unroll
        for (int kk = 0; kk < BC; ++kk) {
            const float *vr = Vs + kk * STR + hf * HALF;
#pragma unroll
            for (int c = 0; c < HALF; ++c) acc[c] = fmaf(s[kk], vr[c], acc[c]);
        }
    }

    if (qrow < N) {
        const float inv = 1.f / l_run;
#pragma unroll
        for (int c4 = 0; c4 < HALF / 4; ++c4) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(acc[4 * c4 + e] * inv);
            buf_store16(w, ro, (uint32_t)(qrow * D + hf * HALF + 4 * c4) * 4u);
        }
        if (hf == 0 && p.lse) p.lse[(size_t)bh * N + qrow] = (m_run + log2f(l_run)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs &a, hipStream_t s) {
    Params p;
    p.q = static_cast<const float *>(a.q);
    p.k = static_cast<const float *>(a.k);
    p.v = static_cast<const float *>(a.v);
    p.o = static_cast<float *>(a.o);
    p.lse = a.lse;
    p.N = a.N;
    p.nqb = (a.N + BR - 1) / BR;
    p.scale_log2 = a.scale * kLog2e;
    const unsigned blocks = (unsigned)a.BH * (unsigned)p.nqb;
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t s) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
    return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace attn
