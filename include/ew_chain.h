/*
 * ew_chain.h -- C ABI of the elementwise-chain fusion example, exported by the
 * same library as attn.h (libattn.so) and using its attn_status codes.
 *
 * The operation ("Attention Is Memory-Bound, and Nobody Noticed for Five
 * Years", the elementwise-chain paragraph: multiply a tensor by a scalar, add
 * a bias, apply an activation; the activation read as ReLU):
 *
 *     y[r, c] = max(scale * x[r, c] + bias[c], 0)
 *
 *   x, y  : bf16 [rows, cols], row-major, no padding; y may equal x (in
 *           place) but may not overlap it otherwise
 *   bias  : float32 [cols]
 *   cols  : a multiple of 8
 * ew_chain_fused computes it in one launch: x is read once and y written
 * once, in fp32 with one rounding to bf16 (nearest even) at the end.
 * ew_chain_unfused is the three-kernel form the page contrasts it with: y =
 * scale * x, then y = y + bias, then y = max(y, 0), each a launch that reads
 * and writes the whole tensor and rounds to bf16.  Both enqueue on `stream`
 * and return; ownership and error conventions are those of attn.h.
 * Checks, in order: rows, cols >= 0 (any zero: ATTN_OK, nothing enqueued)
 * -> NULL x, y, bias (ATTN_ERR_NULL) -> cols % 8 (ATTN_ERR_SHAPE) -> scale
 * finite (ATTN_ERR_ARG) -> x, y, bias 16-byte aligned (ATTN_ERR_ALIGN) ->
 * size -> x and y identical or disjoint, bias not overlapping y
 * (ATTN_ERR_ALIAS).
 */
#ifndef EXACT_ATTENTION_EW_CHAIN_H
#define EXACT_ATTENTION_EW_CHAIN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int ew_chain_fused(const void *x, void *y, const float *bias, long long rows, int cols, float scale,
                   hipStream_t stream);
int ew_chain_unfused(const void *x, void *y, const float *bias, long long rows, int cols, float scale,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* EXACT_ATTENTION_EW_CHAIN_H */
