// C-ABI entry points: argument validation, then one dispatch to the kernel
// launchers.  Nothing here touches the device before validation has passed.
#include <math.h>
#include <stdint.h>

#include "../../include/attn.h"
#include "../../include/ew_chain.h"
#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shared checks of every forward entry point.  Returns ATTN_OK to proceed,
// a negative value for "valid but empty" (nothing to do), or an error code.
// in_elem / out_elem: bytes per element of q, k, v and of o.
int validate_common(const void *q, const void *k, const void *v, const void *o, const float *lse,
                    int B, int H, int N, int d, float scale, int causal, size_t in_elem, size_t out_elem) {
    const size_t elem = in_elem > out_elem ? in_elem : out_elem;
    if (B < 0 || H < 0 || N < 0) return ATTN_ERR_SHAPE;
    if (B == 0 || H == 0 || N == 0) return -1;  // empty: no memory is touched, NULL allowed
    if (!q || !k || !v || !o) return ATTN_ERR_NULL;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_ARG;
    if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ATTN_ERR_ALIGN;
    if (lse && !aligned(lse, 4)) return ATTN_ERR_ALIGN;
    // Per-slice byte offsets are 32-bit inside the kernels (buffer resources),
    // including one padded block of rows past the end.
    const uint64_t slice_bytes = (uint64_t)(N + 2 * attn::kFwdBlockRows) * (uint64_t)d * elem;
    if (slice_bytes >= (1ull << 32)) return ATTN_ERR_SHAPE;
    const uint64_t BH = (uint64_t)B * (uint64_t)H;
    if (BH >= (1ull << 31)) return ATTN_ERR_SHAPE;
    const uint64_t blocks = BH * (uint64_t)((N + attn::kFwdBlockRows - 1) / attn::kFwdBlockRows);
    if (blocks >= (1ull << 31)) return ATTN_ERR_SHAPE;
    const size_t elems = (size_t)BH * (size_t)N * (size_t)d;
    const Range rq = range_of(q, elems * in_elem), rk = range_of(k, elems * in_elem), rv = range_of(v, elems * in_elem);
    const Range ro = range_of(o, elems * out_elem);
    if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv)) return ATTN_ERR_ALIAS;
    if (lse) {
        const Range rl = range_of(lse, (size_t)BH * (size_t)N * sizeof(float));
        if (overlaps(rl, rq) || overlaps(rl, rk) || overlaps(rl, rv) || overlaps(rl, ro)) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

int finish(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

attn::FwdArgs make_args(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                        int N, int d, float scale, int causal) {
    attn::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.BH = B * H;
    a.N = N;
    a.d = d;
    a.scale = scale;
    a.causal = causal;
    return a;
}

int validate_workspace(const void *q, const void *k, const void *v, const void *o, const float *lse,
                       const void *ws, size_t ws_bytes, int B, int H, int N, int d, size_t elem) {
    if (!ws) return ATTN_ERR_NULL;
    const size_t need = attn_unfused_workspace_bytes(B, H, N, (int)elem);
    if (need == 0 || ws_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return ATTN_ERR_ALIGN;
    const size_t tensor = (size_t)B * H * (size_t)N * d * elem;
    const Range rw = range_of(ws, need);
    if (overlaps(rw, range_of(q, tensor)) || overlaps(rw, range_of(k, tensor)) ||
        overlaps(rw, range_of(v, tensor)) || overlaps(rw, range_of(o, tensor)))
        return ATTN_ERR_ALIAS;
    if (lse && overlaps(rw, range_of(lse, (size_t)B * H * (size_t)N * sizeof(float)))) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

// fp8 forward: 1-byte q, k, v and a 2-byte o; the descale factors are
// checked with scale (before alignment, as scale is).
int validate_fp8(const void *q, const void *k, const void *v, const void *o, const float *lse, int B, int H,
                 int N, int d, float scale, float qd, float kd, float vd, int causal) {
    if (B > 0 && H > 0 && N > 0 && q && k && v && o && (d == 64 || d == 128))
        for (float x : {qd, kd, vd})
            if (!isfinite(x) || !(x > 0.f)) return ATTN_ERR_ARG;
    return validate_common(q, k, v, o, lse, B, H, N, d, scale, causal, 1, 2);
}

// Masked forward: bf16 tensors as attn_fwd; the bias must be 4-byte aligned
// with non-negative strides, its per-wave row offsets must fit 32 bits, and
// it must not overlap o or lse.
int validate_masked(const void *q, const void *k, const void *v, const void *o, const float *lse, int B, int H,
                    int N, int d, float scale, int causal, const float *bias, long long sb, long long sh,
                    long long si) {
    const int st = validate_common(q, k, v, o, lse, B, H, N, d, scale, causal, 2, 2);
    if (st != ATTN_OK || !bias) return st;
    if (sb < 0 || sh < 0 || si < 0) return ATTN_ERR_ARG;
    if (!aligned(bias, 4)) return ATTN_ERR_ALIGN;
    if ((32.0 * (double)si + N + 64) * 4.0 >= 4294967296.0) return ATTN_ERR_SHAPE;
    const double ext = (double)(B - 1) * sb + (double)(H - 1) * sh + (double)(N - 1) * si + N;
    if (ext * 4.0 >= 9.0e18) return ATTN_ERR_SHAPE;
    const Range rb = range_of(bias, (size_t)ext * 4);
    const size_t elems = (size_t)B * H * (size_t)N * d;
    if (overlaps(rb, range_of(o, elems * 2))) return ATTN_ERR_ALIAS;
    if (lse && overlaps(rb, range_of(lse, (size_t)B * H * (size_t)N * sizeof(float)))) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

int validate_ew(const void *x, const void *y, const float *bias, long long rows, int cols, float scale) {
    if (rows < 0 || cols < 0) return ATTN_ERR_SHAPE;
    if (rows == 0 || cols == 0) return -1;
    if (!x || !y || !bias) return ATTN_ERR_NULL;
    if (cols % 8) return ATTN_ERR_SHAPE;
    if (!isfinite(scale)) return ATTN_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(bias, 16)) return ATTN_ERR_ALIGN;
    if ((unsigned __int128)rows * (unsigned)cols * 2u >= ((unsigned __int128)1 << 62)) return ATTN_ERR_SHAPE;
    const size_t bytes = (size_t)rows * (size_t)cols * 2;
    const Range rx = range_of(x, bytes), ry = range_of(y, bytes), rb = range_of(bias, (size_t)cols * 4);
    if (x != y && overlaps(rx, ry)) return ATTN_ERR_ALIAS;  // in place is allowed, partial overlap is not
    if (overlaps(rb, ry)) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

// Backward checks.  ws == nullptr with ws_bytes == 0 means "no caller
// workspace" (attn_bwd_noalloc): the workspace null, size, alignment and
// overlap checks are skipped.
int validate_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                 const void *dq, const void *dk, const void *dv, const void *ws, size_t ws_bytes, int B, int H,
                 int N, int d, float scale, int causal, bool caller_workspace) {
    const int st = validate_common(q, k, v, o, lse, B, H, N, d, scale, causal, 2, 2);
    if (st != ATTN_OK) return st;
    if (!lse || !dout || !dq || !dk || !dv || (caller_workspace && !ws)) return ATTN_ERR_NULL;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        (caller_workspace && !aligned(ws, 16)))
        return ATTN_ERR_ALIGN;
    const size_t need = attn_bwd_workspace_bytes(B, H, N);
    if (need == 0 || (caller_workspace && ws_bytes < need)) return ATTN_ERR_WORKSPACE;
    // Grid of the statistics launch: 16 padded rows per workgroup.
    if ((uint64_t)B * H * ((uint64_t)(N + 31) / 32 * 32) / 16 >= (1ull << 31)) return ATTN_ERR_SHAPE;
    const size_t tensor = (size_t)B * H * (size_t)N * d * 2;
    const Range in[6] = {range_of(q, tensor), range_of(k, tensor), range_of(v, tensor), range_of(o, tensor),
                         range_of(dout, tensor), range_of(lse, (size_t)B * H * (size_t)N * sizeof(float))};
    const int nout = caller_workspace ? 4 : 3;
    const Range out[4] = {range_of(dq, tensor), range_of(dk, tensor), range_of(dv, tensor),
                          caller_workspace ? range_of(ws, need) : Range{0, 0}};
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(out[i], in[j])) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(out[i], out[j])) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

attn::BwdArgs make_bwd_args(const void *q, const void *k, const void *v, const void *o, const float *lse,
                            const void *dout, void *dq, void *dk, void *dv, void *workspace, int B, int H, int N,
                            int d, float scale, int causal) {
    attn::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.stats = static_cast<float *>(workspace);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.BH = B * H;
    a.N = N;
    a.d = d;
    a.scale = scale;
    a.causal = causal;
    return a;
}

}  // namespace

extern "C" {

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N, int d,
             float scale, int causal, hipStream_t stream) {
    const int st = validate_common(q, k, v, o, lse, B, H, N, d, scale, causal, 2, 2);
    if (st < 0) return ATTN_OK;
    if (st != ATTN_OK) return st;
    return finish(attn::launch_fwd_bf16(make_args(q, k, v, o, lse, B, H, N, d, scale, causal), stream));
}

int attn_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, int B, int H, int N,
                 int d, float scale, int causal, hipStream_t stream) {
    const int st = validate_common(q, k, v, o, lse, B, H, N, d, scale, causal, 4, 4);
    if (st < 0) return ATTN_OK;
    if (st != ATTN_OK) return st;
    return finish(attn::launch_fwd_f32(make_args(q, k, v, o, lse, B, H, N, d, scale, causal), stream));
}

int attn_fwd_fp8_fmt(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
                     int d, float scale, float q_descale, float k_descale, float v_descale, int q_format,
                     int k_format, int v_format, int causal, hipStream_t stream) {
    const int st = validate_fp8(q, k, v, o, lse, B, H, N, d, scale, q_descale, k_descale, v_descale, causal);
    if (st < 0) return ATTN_OK;
    if (st != ATTN_OK) return st;
    for (int f : {q_format, k_format, v_format})
        if (f != ATTN_FP8_E4M3 && f != ATTN_FP8_E5M2) return ATTN_ERR_ARG;
    attn::Fp8Args a;
    a.f = make_args(q, k, v, o, lse, B, H, N, d, scale, causal);
    a.q_descale = q_descale;
    a.k_descale = k_descale;
    a.v_descale = v_descale;
    a.q_format = q_format;
    a.k_format = k_format;
    a.v_format = v_format;
    return finish(attn::launch_fwd_fp8(a, stream));
}

int attn_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N, int d,
                 float scale, float q_descale, float k_descale, float v_descale, int causal, hipStream_t stream) {
    return attn_fwd_fp8_fmt(q, k, v, o, lse, B, H, N, d, scale, q_descale, k_descale, v_descale, ATTN_FP8_E4M3,
                            ATTN_FP8_E4M3, ATTN_FP8_E4M3, causal, stream);
}

int attn_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N, int d,
                    float scale, int causal, int window_left, int window_right, const float *bias,
                    long long bias_stride_b, long long bias_stride_h, long long bias_stride_i,
                    hipStream_t stream) {
    const int st = validate_masked(q, k, v, o, lse, B, H, N, d, scale, causal, bias, bias_stride_b, bias_stride_h,
                                   bias_stride_i);
    if (st < 0) return ATTN_OK;
    if (st != ATTN_OK) return st;
    attn::MaskedArgs a;
    a.f = make_args(q, k, v, o, lse, B, H, N, d, scale, causal);
    a.H = H;
    a.window_left = window_left < 0 ? -1 : window_left;
    a.window_right = window_right < 0 ? -1 : window_right;
    a.bias = bias;
    a.bias_stride_b = bias_stride_b;
    a.bias_stride_h = bias_stride_h;
    a.bias_stride_i = bias_stride_i;
    return finish(attn::launch_fwd_masked(a, stream));
}

size_t attn_unfused_workspace_bytes(int B, int H, int N, int elem_bytes) {
    if (B <= 0 || H <= 0 || N <= 0 || elem_bytes <= 0) return 0;
    const unsigned __int128 n = (unsigned __int128)B * (unsigned)H * (unsigned)N * (unsigned)N *
                                (unsigned)elem_bytes;
    if (n > (unsigned __int128)SIZE_MAX) return 0;
    return (size_t)n;
}

int attn_fwd_unfused(const void *q, const void *k, const void *v, void *o, float *lse, void *workspace,
                     size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                     hipStream_t stream) {
    int st = validate_common(q, k, v, o, lse, B, H, N, d, scale, causal, 2, 2);
    if (st < 0) return ATTN_OK;
    if (st != ATTN_OK) return st;
    st = validate_workspace(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, 2);
    if (st != ATTN_OK) return st;
    // Score-kernel grid: B*H * ceil(N/128)^2 workgroups.
    const uint64_t nb = (uint64_t)((N + 127) / 128);
    if ((uint64_t)B * H * nb * nb >= (1ull << 31)) return ATTN_ERR_SHAPE;
    return finish(attn::launch_unfused_bf16(make_args(q, k, v, o, lse, B, H, N, d, scale, causal), workspace,
                                            stream));
}

int attn_fwd_unfused_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                         void *workspace, size_t workspace_bytes, int B, int H, int N, int d, float scale,
                         int causal, hipStream_t stream) {
    int st = validate_common(q, k, v, o, lse, B, H, N, d, scale, causal, 4, 4);
    if (st < 0) return ATTN_OK;
    if (st != ATTN_OK) return st;
    st = validate_workspace(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, 4);
    if (st != ATTN_OK) return st;
    const uint64_t nb = (uint64_t)((N + 63) / 64);
    if ((uint64_t)B * H * nb * nb >= (1ull << 31)) return ATTN_ERR_SHAPE;
    return finish(attn::launch_unfused_f32(make_args(q, k, v, o, lse, B, H, N, d, scale, causal), workspace,
                                           stream));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N) {
    if (B <= 0 || H <= 0 || N <= 0) return 0;
    const unsigned __int128 npad = ((unsigned __int128)(unsigned)N + 31) / 32 * 32;
    const unsigned __int128 n = (unsigned __int128)B * (unsigned)H * npad * 2u * 4u;
    if (n > (unsigned __int128)SIZE_MAX) return 0;
    return (size_t)n;
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
             void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes, int B, int H, int N, int d,
             float scale, int causal, hipStream_t stream) {
    if (B < 0 || H < 0 || N < 0) return ATTN_ERR_SHAPE;
    if (B == 0 || H == 0 || N == 0) return ATTN_OK;
    const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, scale,
                                causal, true);
    if (st != ATTN_OK) return st;
    return finish(attn::launch_bwd_bf16(
        make_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale, causal), stream));
}

int attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o, const float *lse,
                     const void *dout, void *dq, void *dk, void *dv, int B, int H, int N, int d, float scale,
                     int causal, hipStream_t stream) {
    static_assert(ATTN_BWD_SCRATCH_BYTES == ((size_t)16 << 20), "header and library must agree");
    if (B < 0 || H < 0 || N < 0) return ATTN_ERR_SHAPE;
    if (B == 0 || H == 0 || N == 0) return ATTN_OK;
    const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, nullptr, 0, B, H, N, d, scale, causal, false);
    if (st != ATTN_OK) return st;
    if (attn_bwd_workspace_bytes(B, H, N) > attn::bwd_scratch_bytes()) return ATTN_ERR_SCRATCH;
    return finish(attn::launch_bwd_bf16_noalloc(
        make_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, nullptr, B, H, N, d, scale, causal), stream));
}

int ew_chain_fused(const void *x, void *y, const float *bias, long long rows, int cols, float scale,
                   hipStream_t stream) {
    const int st = validate_ew(x, y, bias, rows, cols, scale);
    if (st < 0) return ATTN_OK;
    if (st != ATTN_OK) return st;
    return finish(attn::launch_ew_fused(attn::EwArgs{x, y, bias, rows, cols, scale}, stream));
}

int ew_chain_unfused(const void *x, void *y, const float *bias, long long rows, int cols, float scale,
                     hipStream_t stream) {
    const int st = validate_ew(x, y, bias, rows, cols, scale);
    if (st < 0) return ATTN_OK;
    if (st != ATTN_OK) return st;
    return finish(attn::launch_ew_unfused(attn::EwArgs{x, y, bias, rows, cols, scale}, stream));
}

const char *attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "invalid or too large B, H or N";
        case ATTN_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
        case ATTN_ERR_ALIGN: return "misaligned pointer (tensors need 16 bytes, lse 4 bytes)";
        case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
        case ATTN_ERR_WORKSPACE: return "workspace smaller than the matching *_workspace_bytes() reports";
        case ATTN_ERR_HIP: return "HIP runtime error (see attn_last_hip_error)";
        case ATTN_ERR_ARG:
            return "scale and fp8 descale factors must be finite and > 0, causal must be 0 or 1, fp8 formats "
                   "ATTN_FP8_E4M3 or ATTN_FP8_E5M2";
        case ATTN_ERR_SCRATCH:
            return "attn_bwd_noalloc: B*H*round_up(N,32) rows of statistics exceed its static scratch "
                   "(ATTN_BWD_SCRATCH_BYTES); use attn_bwd with a workspace";
        default: return "unknown status";
    }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
