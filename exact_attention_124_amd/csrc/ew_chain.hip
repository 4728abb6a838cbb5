// Elementwise chain y = relu(scale * x + bias), bf16 in/out, gfx950: the
// small fusion example of "Attention Is Memory-Bound, and Nobody Noticed for
// Five Years" (elementwise-chain paragraph).  Run as three kernels, each step
// reads and writes the whole tensor; fused, the tensor is read once and
// written once and the intermediates stay in registers.  Both forms are here
// so the difference can be measured on the same chip.
//
// x and y are [rows, cols] bf16 (row-major, cols a multiple of 8), bias is a
// [cols] fp32 vector added to every row, scale an fp32 scalar.  Every thread
// moves 16-byte chunks (8 elements) with non-temporal loads and stores (the
// tensor is streamed once and should not displace anything in the caches),
// UNROLL chunks in flight per thread; the grid covers the chip a few times
// over and strides through the tensor.  The column of a chunk, needed for the
// bias, is advanced incrementally instead of divided out.
#include "common.h"
#include "launch.h"

namespace attn {
namespace ew {

constexpr int THREADS = 256;
constexpr int UNROLL = 4;

enum Op { FUSED = 0, SCALE = 1, ADD_BIAS = 2, RELU = 3 };

__device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int OP>
__device__ __forceinline__ u32x4 apply(u32x4 v, const float *bias8, float a) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = lo(v[e]);
        f[2 * e + 1] = hi(v[e]);
    }
    if constexpr (OP == FUSED || OP == ADD_BIAS) {
        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bias8);
        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bias8 + 4);
        const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = OP == FUSED ? fmaxf(fmaf(a, f[e], b[e]), 0.f) : f[e] + b[e];
    } else if constexpr (OP == SCALE) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = a * f[e];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = fmaxf(f[e], 0.f);
    }
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
    return out;
}

// n8 = rows * cols / 8 chunks; cols8 = cols / 8.
template <int OP>
__global__ __launch_bounds__(THREADS) void kernel(const u32x4 *x, u32x4 *y, const float *bias, long long n8, int cols8,
                                                  float a) {
    constexpr bool BIAS = OP == FUSED || OP == ADD_BIAS;
    const long long stride = (long long)gridDim.x * THREADS;
    long long i = (long long)blockIdx.x * THREADS + threadIdx.x;
    // Column (in chunks) of chunk i and of the chunks UNROLL strides apart.
    int col = 0, step = 0, ustep = 0;
    if constexpr (BIAS) {
        col = (int)(i % cols8);
        step = (int)(stride % cols8);
        ustep = (int)((stride * UNROLL) % cols8);
    }
    for (; i < n8; i += stride * UNROLL) {
        u32x4 v[UNROLL];
        int c[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const long long j = i + u * stride;
            if (j < n8) v[u] = __builtin_nontemporal_load(x + j);
            if constexpr (BIAS) {
                int cc = col + u * step;
                while (cc >= cols8) cc -= cols8;
                c[u] = cc;
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const long long j = i + u * stride;
            if (j < n8) __builtin_nontemporal_store(apply<OP>(v[u], BIAS ? bias + 8 * c[u] : bias, a), y + j);
        }
        if constexpr (BIAS) {
            col += ustep;
            if (col >= cols8) col -= cols8;
        }
    }
}

template <int OP>
static hipError_t launch(const EwArgs &e, hipStream_t s) {
    const long long n8 = e.rows * (long long)(e.cols / 8);
    const long long want = (n8 + (long long)THREADS * UNROLL - 1) / ((long long)THREADS * UNROLL);
    const unsigned blocks = (unsigned)(want < 256 * 8 ? want : 256 * 8);
    hipLaunchKernelGGL((kernel<OP>), dim3(blocks), dim3(THREADS), 0, s, static_cast<const u32x4 *>(e.x),
                       static_cast<u32x4 *>(e.y), e.bias, n8, e.cols / 8, e.scale);
    return hipGetLastError();
}

}  // namespace ew

hipError_t launch_ew_fused(const EwArgs &e, hipStream_t s) { return ew::launch<ew::FUSED>(e, s); }

// Three launches, each reading and writing the whole tensor; the second and
// third work in place on y.
hipError_t launch_ew_unfused(const EwArgs &e, hipStream_t s) {
    hipError_t r = ew::launch<ew::SCALE>(e, s);
    if (r != hipSuccess) return r;
    EwArgs inplace = e;
    inplace.x = e.y;
    r = ew::launch<ew::ADD_BIAS>(inplace, s);
    if (r != hipSuccess) return r;
    return ew::launch<ew::RELU>(inplace, s);
}

}  // namespace attn
