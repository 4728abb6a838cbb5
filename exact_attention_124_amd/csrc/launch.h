// Internal launch interface between the C-ABI entry points (attn_api.cpp)
// and the kernel translation units.  Every launcher assumes its arguments have
// already been validated by the entry point and returns the hipError_t of the
// launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;  // may be null
    int BH;      // B * H slices
    int N;
    int d;
    float scale;
    int causal;
};

// Fused forward (one kernel launch).
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s);
// Non-causal 8-wave forward (attn_fwd_bf16_dense.hip); called by launch_fwd_bf16.
hipError_t launch_fwd_bf16_dense8(const FwdArgs &a, hipStream_t s);
// Persistent 8-wave forward (attn_fwd_bf16_persistent.hip); called by
// launch_fwd_bf16.  Returns false (launching nothing) when B*H is not a
// multiple of the device's XCD count; else sets err to the launch status.
bool launch_fwd_bf16_persistent(const FwdArgs &a, hipStream_t s, hipError_t &err);
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t s);

// Fused forward on OCP e4m3 inputs with per-tensor dequantisation factors;
// f.o is bf16.
struct Fp8Args {
    FwdArgs f;
    float q_descale;
    float k_descale;
    float v_descale;
    int q_format;  // 0 = OCP e4m3, 1 = OCP e5m2
    int k_format;
    int v_format;
};
hipError_t launch_fwd_fp8(const Fp8Args &a, hipStream_t s);

// Fused forward with a causal / sliding-window mask and an optional fp32
// additive bias (element (b, h, i, j) at bias + b*sb + h*sh + i*si + j).
struct MaskedArgs {
    FwdArgs f;
    int H;
    int window_left;   // < 0: unbounded
    int window_right;  // < 0: unbounded
    const float *bias;
    long long bias_stride_b;
    long long bias_stride_h;
    long long bias_stride_i;
};
hipError_t launch_fwd_masked(const MaskedArgs &a, hipStream_t s);

// Unfused forward: scores -> workspace, softmax in place, probabilities x V.
hipError_t launch_unfused_bf16(const FwdArgs &a, void *ws, hipStream_t s);
hipError_t launch_unfused_f32(const FwdArgs &a, void *ws, hipStream_t s);

struct BwdArgs {
    const void *q;
    const void *k;
    const void *v;
    const void *o;
    const void *dout;
    const float *lse;
    float *stats;  // workspace: BH * 2 * round_up(N, 32) floats
    void *dq;
    void *dk;
    void *dv;
    int BH;
    int N;
    int d;
    float scale;
    int causal;
};

// Backward: row statistics, then dK/dV, then dQ (three launches).
hipError_t launch_bwd_bf16(const BwdArgs &a, hipStream_t s);
// The same launches with the statistics in the library's static per-device
// scratch array (a.stats is ignored); the caller has checked that
// attn_bwd_workspace_bytes() fits bwd_scratch_bytes().
hipError_t launch_bwd_bf16_noalloc(BwdArgs a, hipStream_t s);
size_t bwd_scratch_bytes();

// Elementwise chain y = relu(scale * x + bias) over a [rows, cols] bf16
// tensor (cols a multiple of 8), fused (one launch) or as three launches.
struct EwArgs {
    const void *x;
    void *y;
    const float *bias;  // [cols]
    long long rows;
    int cols;
    float scale;
};
hipError_t launch_ew_fused(const EwArgs &e, hipStream_t s);
hipError_t launch_ew_unfused(const EwArgs &e, hipStream_t s);

// Query-row block of the fused bf16 kernel (used for grid-size limits).
constexpr int kFwdBlockRows = 128;

}  // namespace attn
