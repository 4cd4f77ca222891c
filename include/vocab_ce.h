/*
 * vocab_ce.h -- C ABI of the linear-head cross-entropy over a large
 * vocabulary in libwkv7.so (MI355X, gfx950).
 *
 * The operation. The rwkv-metal page ("Open problems / contributions
 * welcome") asks for the language-model loss over the World vocabulary
 * (65536 entries) to be computed without materialising the [B*T, vocab]
 * logits, by streaming over the vocabulary: an online softmax in the forward
 * and softmax-form gradients in the backward. The rwkv-lab page
 * ("From-scratch pretraining lab", file table) names a fused LM-head
 * cross-entropy with pad masking. For M hidden rows h[m] of width D, a head
 * W with V rows and integer targets t_m:
 *
 *     z[m, v] = sum_d h[m, d] W[v, d]
 *     lse[m]  = log sum_v exp z[m, v]
 *     loss[m] = lse[m] - z[m, t_m]                 (0 for a pad row)
 *     G[m, v] = dloss[m] (exp(z[m, v] - lse[m]) - [v == t_m])   (0 for a pad row)
 *     dh = G W        dW = G^T h
 *
 * A row is a pad row when t_m is outside [0, V) (for example -100). Its lse
 * is still written.
 *
 * Data layout (device memory owned by the caller, row-major, contiguous):
 *   h [M, D] bf16, W [V, D] bf16, targets [M] int32, loss and lse [M] fp32,
 *   dloss [M] fp32, dh [M, D] fp32, dW [V, D] fp32.
 * The products run on bf16 MFMA with fp32 accumulation. G is rounded to bf16
 * before the two gradient products; everything else stays in fp32.
 *
 * Workspace. Both calls take a caller-provided device workspace; the library
 * allocates nothing. The backward processes the vocabulary in chunks of
 * vocab_chunk rows (rounded up to a multiple of 256): its workspace holds the
 * chunk's G in both orders (about 4 * M * vocab_chunk bytes) plus transposed
 * copies of W and h. That is the whole memory floor; the [M, V] logits never
 * exist.
 *
 * Errors. Every argument is checked on the host before anything is
 * enqueued; on an error nothing is launched. Status codes are those of
 * wkv7.h. Work is enqueued on `stream` (a hipStream_t passed as void*; NULL
 * = the null stream) and the call returns without synchronising.
 */
#ifndef VOCAB_CE_H
#define VOCAB_CE_H

#include <stddef.h>
#include <stdint.h>

#include "wkv7.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Sizes accepted by every call: 1 <= M <= 2^28, 64 <= D <= 65536 with D a
 * multiple of 64, 1 <= V <= 2^24, 1 <= vocab_chunk, and no launch of more
 * than 2^22 workgroups: with 256 x 256 tiles, ceil(M/256) * ceil(chunk/256),
 * ceil(M/256) * ceil(D/256) and ceil(chunk/256) * ceil(D/256) are each at
 * most 2^22. Anything else: WKV7_ERR_INVALID_ARGUMENT.
 */

/* Workspace bytes of vce_forward for (M, D, V); *bytes is written on success. */
wkv7_status vce_forward_workspace_bytes(int32_t M, int32_t D, int32_t V, size_t *bytes);

/* Workspace bytes of vce_backward; the vocabulary is processed vocab_chunk rows
 * (rounded up to a multiple of 256, at most V) at a time. */
wkv7_status vce_backward_workspace_bytes(int32_t M, int32_t D, int32_t V, int32_t vocab_chunk,
                                         size_t *bytes);

/*
 * Forward: loss[m] and lse[m] for every row (rwkv-metal, "Open problems /
 * contributions welcome": online softmax over the vocabulary).
 *   h, w      : bf16, 16-byte aligned.
 *   targets   : int32 [M], 4-byte aligned; values outside [0, V) mark pad rows.
 *   loss, lse : fp32 [M] outputs, 4-byte aligned, not overlapping each other.
 *   workspace : >= vce_forward_workspace_bytes, 16-byte aligned, not
 *               overlapping any other argument.
 * Returns WKV7_ERR_WORKSPACE_TOO_SMALL if workspace_bytes is short,
 * WKV7_ERR_UNSUPPORTED if the current device is not gfx950, WKV7_ERR_HIP if
 * a launch fails.
 */
wkv7_status vce_forward(int32_t M, int32_t D, int32_t V, const void *h, const void *w,
                        const int32_t *targets, float *loss, float *lse, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Backward: dh and dW of sum_m dloss[m] loss[m] (rwkv-metal, same section:
 * softmax-form gradients), recomputing the logits from h and W.
 *   lse   : fp32 [M] from vce_forward on the same h, w (pad rows are ignored).
 *   dloss : fp32 [M], the upstream gradient of each row's loss (1/n for a
 *           mean over n unmasked rows).
 *   dh    : fp32 [M, D] output; dw : fp32 [V, D] output (overwritten, not
 *           accumulated into). Neither may overlap an input, each other or
 *           the workspace.
 *   workspace : >= vce_backward_workspace_bytes(M, D, V, vocab_chunk), 16-byte aligned.
 * Errors as for vce_forward.
 */
wkv7_status vce_backward(int32_t M, int32_t D, int32_t V, int32_t vocab_chunk, const void *h,
                         const void *w, const int32_t *targets, const float *lse,
                         const float *dloss, float *dh, float *dw, void *workspace,
                         size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VOCAB_CE_H */
