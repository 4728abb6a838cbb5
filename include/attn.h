/*
 * attn.h -- C ABI of the MI355X (gfx950) exact attention forward library.
 *
 * The operation (grasp.study lesson on standard self-attention, section "The
 * Computational Steps of Standard Self-Attention"; "Attention Is Memory-Bound,
 * and Nobody Noticed for Five Years", exactness paragraphs):
 *
 *     o[b,h,i,:] = sum_j softmax_j( scale * q[b,h,i,:] . k[b,h,j,:] ) * v[b,h,j,:]
 *     lse[b,h,i] = ln sum_j exp( scale * q[b,h,i,:] . k[b,h,j,:] )
 *
 * where j runs over every key (causal = 0) or over j <= i (causal = 1).
 * attn_fwd / attn_fwd_f32 compute it fused, in one kernel per block of query
 * rows: scores, the running (max, sum) softmax and the value weighting stay
 * on chip and only o and lse reach memory ("The Attention Bottleneck -- and How
 * FlashAttention Fixed It", section "The fix: tiling and fusion, never touch
 * HBM").  attn_fwd_unfused / attn_fwd_unfused_f32 compute the same function the
 * standard way, as separate launches that write the N x N score matrix and the
 * probability matrix to device memory and read them back (the trace of a
 * textbook implementation on "Attention Is Memory-Bound ..."): they exist to
 * measure that memory-bound path on the same chip.
 *
 * Layout.  q, k, v and o are dense row-major [B, H, N, d] tensors (d fastest,
 * then N, then H, then B) with no padding between rows; lse is a dense
 * [B, H, N] float array.  The unfused workspace holds one [B, H, N, N] matrix.
 *
 * Ownership.  Every pointer is a device pointer owned by the caller, who
 * allocates and frees it.  The library allocates, frees and synchronises
 * nothing; it only enqueues kernels on `stream` (0 = the null stream) and
 * returns.  Errors raised while the kernels run surface at the caller's next
 * synchronisation of that stream.
 *
 * Errors.  Arguments are validated, in the order listed on each function,
 * before any HIP call.  A failing check returns its status code and enqueues
 * nothing; there is never a silent fallback to another algorithm.  A HIP
 * launch failure returns ATTN_ERR_HIP; attn_last_hip_error() then gives the
 * hipError_t for the calling thread.  No C++ exception crosses this ABI.  All
 * calls are thread-safe (the only mutable state is the thread-local error).
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,      /* a required pointer is NULL                                 */
    ATTN_ERR_SHAPE = 2,     /* B, H or N negative, or a size limit below exceeded          */
    ATTN_ERR_HEAD_DIM = 3,  /* d is not 64 or 128                                         */
    ATTN_ERR_ALIGN = 4,     /* q, k, v, o or workspace not 16-byte aligned; lse not 4-byte */
    ATTN_ERR_ALIAS = 5,     /* an output range overlaps an input or another output range   */
    ATTN_ERR_WORKSPACE = 6, /* workspace smaller than attn_unfused_workspace_bytes / attn_bwd_workspace_bytes */
    ATTN_ERR_HIP = 7,       /* a HIP runtime call failed (see attn_last_hip_error)        */
    ATTN_ERR_ARG = 8,       /* scale (or an fp8 descale) not finite and > 0, causal not 0/1, or an unknown fp8 format */
    ATTN_ERR_SCRATCH = 9    /* attn_bwd_noalloc: the statistics exceed the library's static scratch */
} attn_status;

/*
 * Fused forward, bfloat16.
 *   q, k, v : const bf16 [B,H,N,d] inputs (raw 16-bit bfloat16 words)
 *   o       : bf16 [B,H,N,d] output, rounded to nearest even from fp32
 *   lse     : float [B,H,N] natural-log log-sum-exp of the scaled, masked
 *             scores, or NULL to skip it
 *   scale   : multiplies q.k (usually 1/sqrt(d)); must be finite and > 0
 *   causal  : 0 = every key, 1 = key j allowed for query i iff j <= i
 * Products accumulate in fp32 on the matrix cores; the softmax runs in fp32
 * with base-2 exponentials; the probabilities feed the second product as bf16.
 * Checks, in order: B,H,N >= 0 (any zero: return ATTN_OK, nothing enqueued,
 * pointers may then be NULL) -> NULL (q,k,v,o) -> d in {64,128} -> scale,
 * causal -> alignment -> limits ((N+256)*d*elem_bytes < 2^32 per slice,
 * B*H < 2^31, workgroups < 2^31) -> o and lse do not overlap q, k, v or each
 * other.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Fused forward, float32 in and out, fp32 arithmetic throughout (vector
 * units, no reduced-precision step).  Same parameters and checks as attn_fwd. */
int attn_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                 int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Fused forward on 8-bit floating-point inputs: the low-precision variant
 * that "Attention Is Memory-Bound, and Nobody Noticed for Five Years"
 * reports for the FlashAttention-3 generation (results paragraph), computing
 * the attn_fwd function of the dequantised inputs
 *     Q = q_descale * q,   K = k_descale * k,   V = v_descale * v.
 *   q, k, v : const [B,H,N,d] bytes in the OCP FP8 E4M3 format (1 sign bit,
 *             4 exponent bits with bias 7, 3 mantissa bits; subnormals; no
 *             infinities; 0x7F and 0xFF are NaN, which the caller must not
 *             pass; largest finite value 448)
 *   o       : bf16 [B,H,N,d] output (real scale, RNE from fp32)
 *   lse     : float [B,H,N] natural-log log-sum-exp of the real scaled scores
 *             (scale * Q.K), or NULL
 *   q_descale, k_descale, v_descale : per-tensor dequantisation factors,
 *             finite and > 0
 * Both products run on the fp8 matrix-core instructions with fp32
 * accumulation; the softmax is fp32; the probabilities are rounded to E4M3
 * (nearest even, values at most 2^8) before the second product.
 * Checks: as attn_fwd (alignment 16 bytes for q, k, v and o; per-slice limit
 * (N+256)*d*2 < 2^32), with the three descale factors checked with scale.
 */
int attn_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int H, int N, int d, float scale,
                 float q_descale, float k_descale, float v_descale, int causal, hipStream_t stream);

/* 8-bit formats of attn_fwd_fp8_fmt's inputs. */
enum { ATTN_FP8_E4M3 = 0, ATTN_FP8_E5M2 = 1 };

/*
 * attn_fwd_fp8 with the 8-bit format of each input chosen separately:
 * q_format, k_format, v_format each ATTN_FP8_E4M3 (as attn_fwd_fp8) or
 * ATTN_FP8_E5M2, the OCP FP8 E5M2 format (1 sign bit, 5 exponent bits with
 * bias 15, 2 mantissa bits; subnormals; 0x7C and 0xFC are infinities and
 * 0x7D-0x7F, 0xFD-0xFF NaN, which the caller must not pass; largest finite
 * value 57344).  The function computed is the same (the inputs dequantised
 * from their formats); the probabilities are still rounded to E4M3 before
 * the second product.  Checks: as attn_fwd_fp8; a format other than the two
 * returns ATTN_ERR_ARG.  attn_fwd_fp8 is this call with all three formats
 * ATTN_FP8_E4M3.
 */
int attn_fwd_fp8_fmt(const void *q, const void *k, const void *v, void *o, float *lse,
                     int B, int H, int N, int d, float scale,
                     float q_descale, float k_descale, float v_descale,
                     int q_format, int k_format, int v_format, int causal, hipStream_t stream);

/*
 * Fused forward with a general mask and an additive bias, bfloat16: the
 * custom masks and attention biases that the pages name as what usually
 * takes attention off the fused path ("Attention Is Memory-Bound, and Nobody
 * Noticed for Five Years", the paragraph on what the result means in
 * practice), computed on it:
 *     s[b,h,i,j] = scale * q[b,h,i,:] . k[b,h,j,:] + bias[b,h,i,j]
 * over the keys j allowed for query i, softmax over them, times v.
 *   causal        : 0/1, as attn_fwd
 *   window_left   : key j allowed only if j >= i - window_left (< 0: no limit)
 *   window_right  : key j allowed only if j <= i + window_right (< 0: no limit)
 *   bias          : NULL, or float32 with element (b,h,i,j) at
 *                   bias[b*bias_stride_b + h*bias_stride_h + i*bias_stride_i + j]
 *                   (strides in elements, >= 0; 0 broadcasts over that
 *                   index); -inf removes a key (a boolean mask).  A bias
 *                   16-byte aligned with strides that are multiples of 4 is
 *                   read 16 bytes at a time, any other 4 bytes at a time
 * A query row with no allowed key of finite score gets o = 0 and lse = -inf.
 * Key tiles outside a workgroup's allowed range are skipped, so a sliding
 * window costs work proportional to its width.
 * Checks: as attn_fwd, then (bias only) strides >= 0 (ATTN_ERR_ARG), bias
 * 4-byte aligned (ATTN_ERR_ALIGN),
 * (32*bias_stride_i + N + 64)*4 < 2^32 (ATTN_ERR_SHAPE), and the bias extent
 * not overlapping o or lse (ATTN_ERR_ALIAS).
 */
int attn_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int N, int d, float scale, int causal,
                    int window_left, int window_right, const float *bias,
                    long long bias_stride_b, long long bias_stride_h, long long bias_stride_i,
                    hipStream_t stream);

/* Bytes of workspace the unfused variant needs: B*H*N*N*elem_bytes
 * (elem_bytes = 2 for attn_fwd_unfused, 4 for attn_fwd_unfused_f32).  Returns
 * 0 for non-positive arguments or on size_t overflow.  Pure host function. */
size_t attn_unfused_workspace_bytes(int B, int H, int N, int elem_bytes);

/*
 * Unfused forward, bfloat16: three launches on `stream`.
 *   1. scores: workspace <- q k^T (raw dot products, rounded to bf16)
 *   2. softmax: per row, scale, mask, subtract the max, exponentiate,
 *      normalise; the bf16 probabilities overwrite the scores in place; lse
 *   3. output: o <- P v
 * workspace: device buffer of at least attn_unfused_workspace_bytes(B,H,N,2)
 * bytes, 16-byte aligned, not overlapping q, k, v, o or lse; its contents on
 * return are the probabilities P [B,H,N,N].
 * Checks: as attn_fwd, then workspace NULL (ATTN_ERR_NULL), size
 * (ATTN_ERR_WORKSPACE), alignment and overlap.
 */
int attn_fwd_unfused(const void *q, const void *k, const void *v, void *o, float *lse,
                     void *workspace, size_t workspace_bytes,
                     int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Unfused forward, float32 scores and probabilities (workspace elem_bytes 4). */
int attn_fwd_unfused_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                         void *workspace, size_t workspace_bytes,
                         int B, int H, int N, int d, float scale, int causal,
                         hipStream_t stream);

/*
 * Backward of the fused forward, bfloat16: gradients of the attention output
 * with respect to q, k and v for an upstream gradient dout, computed the same
 * fused way (the N x N probabilities are recomputed tile by tile from q, k and
 * the forward's lse and never stored).  The function differentiated is the
 * one attn_fwd computes (grasp.study lesson on standard self-attention,
 * section "The Computational Steps of Standard Self-Attention"; the pages
 * report the fused method's training speed in "Attention Is Memory-Bound, and
 * Nobody Noticed for Five Years", results paragraph, but do not write out the
 * gradient):
 *     dV = P^T dO,   dS = P o (dO V^T - rowsum(dO o O)),
 *     dQ = scale dS K,   dK = scale dS^T Q.
 *   q, k, v, o, dout : const bf16 [B,H,N,d]; o and lse are attn_fwd's outputs
 *                      for these q, k, v, scale and causal (not checked)
 *   lse              : const float [B,H,N], required
 *   dq, dk, dv       : bf16 [B,H,N,d] outputs (RNE from fp32)
 *   workspace        : device buffer of at least attn_bwd_workspace_bytes()
 *                      bytes, 16-byte aligned; holds per-row statistics
 * Three launches on `stream`; the result is deterministic (no atomics).
 * Checks: as attn_fwd (with dout, dq, dk, dv, lse and workspace required and
 * aligned), workspace size (ATTN_ERR_WORKSPACE), and no output or workspace
 * range overlapping an input range or another output (ATTN_ERR_ALIAS).
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dout, void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
             int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Workspace bytes attn_bwd needs: B*H*2*round_up(N, 32)*4.  Returns 0 for
 * non-positive arguments or on size_t overflow.  Pure host function. */
size_t attn_bwd_workspace_bytes(int B, int H, int N);

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The per-row statistics go to a static device array
 * inside the library (ATTN_BWD_SCRATCH_BYTES per GPU, held until the process
 * ends); nothing is allocated or freed by the call.
 *   Arguments, layouts, results and the other checks are those of attn_bwd.
 *   The statistics need attn_bwd_workspace_bytes(B, H, N) bytes; a problem
 *   needing more than ATTN_BWD_SCRATCH_BYTES returns ATTN_ERR_SCRATCH and
 *   enqueues nothing (B*H*round_up(N, 32) <= 2^21 rows fits, e.g.
 *   8 x 32 x 8192).
 *   On its first call on a device the library looks up that device's copy of
 *   the array (hipGetSymbolAddress, with the device current); a failure there
 *   returns ATTN_ERR_HIP.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents: calls that overlap on one GPU (on different streams, or
 *   from several threads without ordering) race on it and their results are
 *   undefined.  Calls ordered on one stream are safe.
 */
#define ATTN_BWD_SCRATCH_BYTES ((size_t)16 << 20)
int attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o, const float *lse,
                     const void *dout, void *dq, void *dk, void *dv,
                     int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Static text for a status code ("unknown status" for anything else). */
const char *attn_status_string(int status);

/* hipError_t of the calling thread's last ATTN_ERR_HIP (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* EXACT_ATTENTION_ATTN_H */
