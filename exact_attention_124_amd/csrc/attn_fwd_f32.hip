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
    int xcds;  // L2 domains of the device (block remap)
};

constexpr int BR = 128;  // query rows per workgroup
constexpr int BC = 32;   // keys per tile

// Running state of one (row, half of d) lane: the row's running maximum of
// the base-2 logits, the running sum of exponentials, and its half of the
// unnormalised output.
template <int D>
struct RowState {
    float acc[D / 2];
    float m_run, l_run;
};

template <int D>
__device__ __forceinline__ void init_state(RowState<D> &st) {
#pragma unroll
    for (int c = 0; c < D / 2; ++c) st.acc[c] = 0.f;
    st.m_run = -INFINITY;
    st.l_run = 0.f;
}

// One tile of BC keys starting at key0, whose K and V rows sit in LDS at kt
// and vt (row stride STR floats): scores, the tile's row maximum, the
// rescale of the running state, and the weighted V rows.  Keys past `lim`
// (the last key the row may see) score -inf.
template <int D, bool CAUSAL>
__device__ __forceinline__ void tile_update(RowState<D> &st, const float *qv, const float *kt,
                                            const float *vt, int key0, int lim, bool edge, int hf,
                                            float cl) {
    constexpr int HALF = D / 2;
    constexpr int STR = D + 4;
    float s[BC];
#pragma unroll
    for (int kk = 0; kk < BC; ++kk) {
        const float *kr = kt + kk * STR + hf * HALF;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < HALF; ++c) part = fmaf(qv[c], kr[c], part);
        s[kk] = pair_sum(part);
    }
    if (edge) {
#pragma unroll
        for (int kk = 0; kk < BC; ++kk)
            if (key0 + kk > lim) s[kk] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int kk = 1; kk < BC; ++kk) mx = fmaxf(mx, s[kk]);
    const float m_new = fmaxf(st.m_run, mx * cl);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(st.m_run - m_use);
    st.m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kk = 0; kk < BC; ++kk) {
        s[kk] = exp2f(fmaf(s[kk], cl, -m_use));
        rs += s[kk];
    }
    st.l_run = st.l_run * alpha + rs;
#pragma unroll
    for (int c = 0; c < HALF; ++c) st.acc[c] *= alpha;
#pragma unroll
    for (int kk = 0; kk < BC; ++kk) {
        const float *vr = vt + kk * STR + hf * HALF;
#pragma unroll
        for (int c = 0; c < HALF; ++c) st.acc[c] = fmaf(s[kk], vr[c], st.acc[c]);
    }
}

// Q row (this lane's half of it) into registers; rows >= N read as zero.
template <int D>
__device__ __forceinline__ void load_q_half(float *qv, __amdgpu_buffer_rsrc_t rq, int qrow, int hf) {
    constexpr int HALF = D / 2;
#pragma unroll
    for (int c4 = 0; c4 < HALF / 4; ++c4) {
        const u32x4 x = buf_load16(rq, (uint32_t)(qrow * D + hf * HALF + 4 * c4) * 4u);
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[4 * c4 + e] = __uint_as_float(x[e]);
    }
}

// rows x D floats from `r` starting at row `row0` into LDS (stride STR);
// rows >= N read as zero.
template <int D, int ROWS>
__device__ __forceinline__ void stage_rows(float *dst, __amdgpu_buffer_rsrc_t r, int row0, int tid) {
    constexpr int STR = D + 4;
    for (int ch = tid; ch < ROWS * D / 4; ch += 256) {
        const int row = ch / (D / 4), col4 = ch % (D / 4);
        const uint32_t off = (uint32_t)((row0 + row) * D + 4 * col4) * 4u;
        *reinterpret_cast<u32x4 *>(dst + row * STR + 4 * col4) = buf_load16(r, off);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(Params p) {
    constexpr int HALF = D / 2;
    constexpr int STR = D + 4;  // LDS row stride (floats)
    __shared__ __attribute__((aligned(16))) float Ks[BC * STR];
    __shared__ __attribute__((aligned(16))) float Vs[BC * STR];

    const int logical = xcd_remap(blockIdx.x, gridDim.x, p.xcds);
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
    load_q_half<D>(qv, rq, qrow, hf);
    RowState<D> st;
    init_state<D>(st);
    const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;

    int ntiles = (N + BC - 1) / BC;
    if (CAUSAL) ntiles = min(ntiles, (qb * BR + BR + BC - 1) / BC);

    for (int j = 0; j < ntiles; ++j) {
        const int key0 = j * BC;
        __syncthreads();  // previous tile fully consumed
        stage_rows<D, BC>(Ks, rk, key0, tid);
        stage_rows<D, BC>(Vs, rv, key0, tid);
        __syncthreads();
        if (CAUSAL && key0 > q0 + 31) continue;  // whole tile masked for this wave
        const bool edge = (CAUSAL && key0 + BC - 1 > q0) || key0 + BC > N;
        tile_update<D, CAUSAL>(st, qv, Ks, Vs, key0, lim, edge, hf, p.scale_log2);
    }

    if (qrow < N) {
        const float inv = 1.f / st.l_run;
#pragma unroll
        for (int c4 = 0; c4 < HALF / 4; ++c4) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(st.acc[4 * c4 + e] * inv);
            buf_store16(w, ro, (uint32_t)(qrow * D + hf * HALF + 4 * c4) * 4u);
        }
        if (hf == 0 && p.lse) p.lse[(size_t)bh * N + qrow] = (st.m_run + log2f(st.l_run)) * kLn2;
    }
}

// Split-key variant for grids too small to occupy the chip: a workgroup owns
// 32 query rows and its four waves take the four 32-key quarters of each
// 128-key step, each keeping its own running state (the running
// normalisation of "The Attention Bottleneck -- and How FlashAttention Fixed
// It", section "The fix: tiling and fusion, never touch HBM").  At the end the
// four states of a row are merged under their common maximum,
//     m = max_w m_w,  l = sum_w 2^(m_w - m) l_w,  O = sum_w 2^(m_w - m) O_w / l,
// which gives the same result as one pass over all keys up to rounding: each
// state's sum and output were accumulated relative to its own m_w, and the
// factor 2^(m_w - m) moves them to the common reference.  (The pages do not
// state this merge; it follows from the definition of the softmax.)
constexpr int SPLIT = 4;  // waves per query block, one per key quarter

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_f32_split_kernel(Params p) {
    constexpr int HALF = D / 2;
    constexpr int STR = D + 4;
    constexpr int STEP = SPLIT * BC;          // keys per barrier step
    constexpr int SLOT = 64 * (HALF + 2);     // floats of one wave's state
    static_assert(SPLIT * SLOT <= STEP * STR, "merge area must fit in the K buffer");
    __shared__ __attribute__((aligned(16))) float Ks[STEP * STR];
    __shared__ __attribute__((aligned(16))) float Vs[STEP * STR];

    const int logical = xcd_remap(blockIdx.x, gridDim.x, p.xcds);
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

    const int q0 = qb * 32;
    const int qrow = q0 + l32;

    float qv[HALF];
    load_q_half<D>(qv, rq, qrow, hf);
    RowState<D> st;
    init_state<D>(st);
    const int lim = CAUSAL ? min(qrow, N - 1) : N - 1;

    const int last_key = CAUSAL ? min(q0 + 31, N - 1) : N - 1;
    const int nsteps = last_key / STEP + 1;
    for (int j = 0; j < nsteps; ++j) {
        const int step0 = j * STEP;
        __syncthreads();
        stage_rows<D, STEP>(Ks, rk, step0, tid);
        stage_rows<D, STEP>(Vs, rv, step0, tid);
        __syncthreads();
        const int key0 = step0 + wave * BC;
        if (key0 > last_key) continue;  // every key of this quarter is masked
        const bool edge = (CAUSAL && key0 + BC - 1 > q0) || key0 + BC > N;
        tile_update<D, CAUSAL>(st, qv, Ks + wave * BC * STR, Vs + wave * BC * STR, key0, lim,
                               edge, hf, p.scale_log2);
    }

    // Merge.  Wave w leaves its state in slot w of the (now free) K buffer:
    // per lane HALF outputs then m and l, lane-major so that the combining
    // reads below are lane-contiguous.
    __syncthreads();
    float *mine = Ks + wave * SLOT;
#pragma unroll
    for (int c = 0; c < HALF; ++c) mine[c * 64 + lane] = st.acc[c];
    mine[HALF * 64 + lane] = st.m_run;
    mine[(HALF + 1) * 64 + lane] = st.l_run;
    __syncthreads();

    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < SPLIT; ++w) m = fmaxf(m, Ks[w * SLOT + HALF * 64 + lane]);
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float f[SPLIT];
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < SPLIT; ++w) {
        f[w] = exp2f(Ks[w * SLOT + HALF * 64 + lane] - m_use);
        l += f[w] * Ks[w * SLOT + (HALF + 1) * 64 + lane];
    }
    // Wave t writes columns [t * HALF/4, (t+1) * HALF/4) of this lane's half.
    constexpr int PART = HALF / SPLIT;
    if (qrow < N) {
        const float inv = 1.f / l;
#pragma unroll
        for (int c4 = 0; c4 < PART / 4; ++c4) {
            u32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = wave * PART + 4 * c4 + e;
                float x = 0.f;
#pragma unroll
                for (int w = 0; w < SPLIT; ++w) x = fmaf(f[w], Ks[w * SLOT + c * 64 + lane], x);
                out[e] = __float_as_uint(x * inv);
            }
            buf_store16(out, ro, (uint32_t)(qrow * D + hf * HALF + wave * PART + 4 * c4) * 4u);
        }
        if (wave == 0 && hf == 0 && p.lse) p.lse[(size_t)bh * N + qrow] = (m_use + log2f(l)) * kLn2;
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
    const DeviceShape shape = device_shape();
    p.xcds = shape.xcds;
    const long long blocks = (long long)a.BH * p.nqb;
    if (blocks < shape.cus) {
        // Fewer workgroups than compute units: four times as many, each
        // splitting its keys over its waves.
        p.nqb = (a.N + 31) / 32;
        hipLaunchKernelGGL((attn_fwd_f32_split_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * p.nqb)),
                           dim3(256), 0, s, p);
    } else {
        hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, s,
                           p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t s) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, s) : launch<128, false>(a, s);
    return a.causal ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace attn
