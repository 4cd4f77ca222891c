/*
 * wkv7.h -- C ABI of libwkv7.so, the MI355X (gfx950) WKV-7 recurrence library.
 *
 * The operation (RWKV-7 "Goose" WKV-7, the recurrence the rwkv-metal page's
 * section "The Metal WKV-7 kernel" and the model card's "Transformers
 * quickstart" section describe as the one custom kernel of the model): per
 * independent unit -- one (sequence, head) pair -- with head size N = 64 (the
 * forward, the backward and the decode steps also take N = 128) and an fp32 state S in
 * R^{NxN} indexed [value i, key j], every token t does
 *
 *     S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T + v_t k_t^T,   y_t = S_t r_t
 *
 * where the a-term reads the undecayed S_{t-1} and y_t reads the updated S_t.
 *
 * Data layout (all buffers are device memory owned by the caller):
 *   token streams r, w, k, v, a, b, y, dy, dr..db : [B, T, H, N], N contiguous,
 *       element type given by wkv7_desc.dtype (fp32, bf16 or fp16: the model
 *       card's "Transformers quickstart" section names BF16/FP16/FP32
 *       activations); dr..db in fp32 instead when wkv7_desc.grad_f32 = 1;
 *       the flat token index of (row b, position t) is b*T + t;
 *   states s0, s_out, ds_out, ds0 : fp32 [S, H, N, N], row = value index i,
 *       column = key index j; S = B in dense mode, num_seqs in segment mode;
 *   checkpoints ckpt : fp32 [slots, H, N, N]; the checkpoint of chunk c of a
 *       sequence (the state entering its token 16c, so chunk 0 holds its
 *       initial state) sits at slot base + c, where base = b*ceil(T/16) for
 *       dense row b and base = seq_ckpt[s] for sequence s in segment mode.
 *       The state is checkpointed every 16 tokens as on the rwkv-metal page
 *       (section "The Metal WKV-7 kernel") and the RWKV-MLX page (section
 *       "Key Design Decisions", CHUNK_LEN=16 backward).
 *
 * Decay input. With wkv7_desc.decay = WKV7_DECAY_MULT the w stream holds the
 * multiplicative decay itself (in [0, 1]). With WKV7_DECAY_LOG it holds its
 * natural logarithm and the decay is exp(w) (w <= 0), the form in which the
 * wkv7 call on the rwkv-lab page (section "Highlight result -- GDN in RWKV-7")
 * takes GDN's log-decay; dw is then the gradient with respect to that
 * logarithm, i.e. decay * dL/d(decay).
 *
 * Modes.
 *   Dense (num_seqs == 0): each of the B rows is one sequence of T tokens.
 *   Segment (num_seqs > 0): sequence s covers flat tokens
 *       [seq_start[s], seq_start[s] + seq_len[s]), which must lie inside one
 *       row; sequences must not overlap. Each sequence starts from its own
 *       initial state (s0[s], or zero), so nothing crosses a boundary: this
 *       serves packed streams with a state reset at every boundary (rwkv-lab
 *       page, post-training trainer paragraph; model card, "Transformers
 *       quickstart") and right-padded ragged rows (rwkv-metal page,
 *       feature list). Tokens covered by no sequence are never read; the
 *       forward writes y = 0 there and the backward writes zero gradients.
 *   Any T >= 1 is accepted (no padding to a multiple of 16 is needed).
 *
 * Ownership and threading. The library allocates no device memory in these
 * calls and keeps no pointer after return. Work is enqueued on `stream` (a
 * hipStream_t passed as void*; NULL = the null stream) and the call returns
 * without synchronising. Calls are thread-safe.
 *
 * Errors. Arguments are validated on the host before anything is enqueued;
 * on any error nothing is launched. Segment tables live in device memory and
 * cannot be checked by the host: wkv7_segments_check validates a host copy.
 * The kernels skip (leave as zero) any sequence whose entry is out of range
 * instead of touching memory outside the buffers. No C++ exception crosses
 * this boundary.
 */
#ifndef WKV7_H
#define WKV7_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WKV7_ABI_VERSION 2
#define WKV7_HEAD_SIZE 64        /* the head size every call takes */
#define WKV7_HEAD_SIZE_WIDE 128  /* also taken by wkv7_forward, wkv7_backward,
                                    wkv7_workspace_bytes, wkv7_decode_step and
                                    the gated DeltaNet calls */
#define WKV7_CHUNK 16
/* static scratch of wkv7_backward_noalloc per device: 128 MiB, enough for
   B*ceil(T/16)*H <= 6241 (e.g. B=1, T=3120, H=32) */
#define WKV7_STATIC_SCRATCH_BYTES ((size_t)128 << 20)

typedef enum {
    WKV7_OK = 0,
    WKV7_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad size, bad table */
    WKV7_ERR_UNSUPPORTED = 2,        /* e.g. a head size the call does not take, unknown dtype, no gfx950 device */
    WKV7_ERR_WORKSPACE_TOO_SMALL = 3,
    WKV7_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} wkv7_status;

typedef enum {
    WKV7_F32 = 0,
    WKV7_BF16 = 1,
    WKV7_F16 = 2
} wkv7_dtype;

typedef enum {
    WKV7_DECAY_MULT = 0,        /* w is the decay */
    WKV7_DECAY_LOG = 1          /* w is log(decay); decay = exp(w) */
} wkv7_decay;

typedef struct {
    int32_t B;                  /* rows */
    int32_t T;                  /* tokens per row, >= 1 */
    int32_t H;                  /* heads, 1 <= H <= 65536 */
    int32_t N;                  /* head size: 64, or 128 (wkv7_forward, wkv7_backward) */
    int32_t dtype;              /* wkv7_dtype of r,w,k,v,a,b,y,dy and dr..db */
    int32_t num_seqs;           /* 0 = dense mode */
    const int32_t *seq_start;   /* device [num_seqs]: flat start token b*T + t */
    const int32_t *seq_len;     /* device [num_seqs]: length >= 0 */
    const int32_t *seq_ckpt;    /* device [num_seqs]: first checkpoint slot; needed
                                   only when checkpoints are written or read */
    int32_t ckpt_slots;         /* segment mode: slots in the ckpt buffer */
    int32_t decay;              /* wkv7_decay of the w stream (0 = multiplicative) */
    int32_t grad_f32;           /* 1: dr..db are fp32 whatever dtype is; 0: dtype */
} wkv7_desc;

/*
 * Forward over a batch: y (and optionally s_out, ckpt) from r..b and s0.
 *   r, w, k, v, a, b : [B,T,H,N] inputs; w is the multiplicative decay.
 *   s0    : [S,H,N,N] fp32 initial states, or NULL for zeros.
 *   y     : [B,T,H,N] output (dtype); required.
 *   s_out : [S,H,N,N] fp32 final states, or NULL.
 *   ckpt  : [slots,H,N,N] fp32 checkpoints for wkv7_backward, or NULL
 *           (inference forward). Dense mode needs B*ceil(T/16) slots.
 * All pointers 16-byte aligned. No output (y, s_out, ckpt) may share a byte
 * with an input or another output: WKV7_ERR_INVALID_ARGUMENT.
 */
wkv7_status wkv7_forward(const wkv7_desc *d,
                         const void *r, const void *w, const void *k,
                         const void *v, const void *a, const void *b,
                         const float *s0, void *y, float *s_out, float *ckpt,
                         void *stream);

/*
 * Backward: gradients of L = sum <dy, y> + <ds_out, S_T> with respect to
 * r, w, k, v, a, b (written in dtype) and the initial state (fp32).
 *   ckpt   : checkpoints written by wkv7_forward on the same inputs and s0.
 *   dy     : [B,T,H,N] upstream gradient of y (dtype), or NULL for zero.
 *   ds_out : [S,H,N,N] fp32 upstream gradient of the final state, or NULL.
 *   dr..db : [B,T,H,N] outputs (dtype, or fp32 when grad_f32 = 1); required.
 *   ds0    : [S,H,N,N] fp32 gradient of the initial state, or NULL.
 *   workspace / workspace_bytes : device memory of at least
 *           wkv7_workspace_bytes, 16-byte aligned, owned by the caller. The
 *           call overwrites it with fp32 per-chunk results of the first
 *           kernel (the gradient of the state leaving each 16-token chunk,
 *           64x64; the chunk's 16x16 inverse W of its unit-lower triangular
 *           system; and the 16x64 product of W's transpose with the chunk's
 *           gradient of that system's solution; per checkpoint slot and
 *           head; the first and third in bf16 when the streams and the
 *           gradients are bf16) and reads them back within the same call; calls that may run
 *           concurrently need separate workspaces. Too small or NULL when
 *           needed: WKV7_ERR_WORKSPACE_TOO_SMALL, before any HIP call.
 * No output (dr..db, ds0, workspace) may share a byte with an input (r..b,
 * ckpt, dy, ds_out) or another output: WKV7_ERR_INVALID_ARGUMENT.
 * The recurrence is recomputed from the 16-token checkpoints in fp32, not
 * reconstructed by dividing by the decay. N = 64: two kernels run back to
 * back on `stream`, a reverse sweep that carries only the state gradient,
 * then the per-chunk gradients, all chunks in parallel; with bf16 streams
 * the second kernel's products run on bf16 MFMA with fp32 accumulation, each
 * operand rounded to one bf16 piece for bf16 gradients (the order of the
 * gradients' own bf16 rounding) and split into two pieces (about 2^-16
 * relative) when grad_f32 = 1. N = 128: token by
 * token, one workgroup per (sequence, head) through the whole sequence in
 * reverse, every gradient summed within the workgroup (no workspace; the
 * results do not depend on scheduling).
 */
wkv7_status wkv7_backward(const wkv7_desc *d,
                          const void *r, const void *w, const void *k,
                          const void *v, const void *a, const void *b,
                          const float *ckpt, const void *dy, const float *ds_out,
                          void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                          float *ds0, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * wkv7_backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments and results are those of wkv7_backward, without the workspace:
 * the per-chunk results of the first kernel go to a static device array of
 * WKV7_STATIC_SCRATCH_BYTES that the library holds on every device it runs
 * on until the process ends. A descriptor whose wkv7_workspace_bytes exceeds
 * that size gets WKV7_ERR_WORKSPACE_TOO_SMALL before any HIP call. The call
 * allocates nothing; its first call on a device looks up the array's address
 * there. Every call on one device uses the same array, and each call writes
 * every entry it reads before reading it: calls that may overlap in time on
 * one device (on different streams, or from several threads) race and must
 * be serialised by the caller. Head size 64 only (N = 128:
 * WKV7_ERR_UNSUPPORTED).
 */
wkv7_status wkv7_backward_noalloc(const wkv7_desc *d,
                                  const void *r, const void *w, const void *k,
                                  const void *v, const void *a, const void *b,
                                  const float *ckpt, const void *dy, const float *ds_out,
                                  void *dr, void *dw, void *dk, void *dv, void *da, void *db,
                                  float *ds0, void *stream);

/*
 * One decode step for B independent sequences (the rwkv-metal page's
 * wkv7_step; the rwkv-lab page's in-place one-token state transition).
 *   N     : head size, 64, or 128 (the matched head size of the rwkv-lab
 *           page's GDN conversion target); anything else: WKV7_ERR_UNSUPPORTED.
 *   dtype : wkv7_dtype of r..b and y; decay : wkv7_decay of w.
 *   r..b  : [B,H,N] one token per sequence (dtype).
 *   s_in  : [B,H,N,N] fp32 state before the token.
 *   s_out : [B,H,N,N] fp32 state after the token; may equal s_in (in place),
 *           otherwise must not overlap it.
 *   y     : [B,H,N] output (dtype).
 * Apart from s_out == s_in, no output (s_out, y) may share a byte with an
 * input or the other output: WKV7_ERR_INVALID_ARGUMENT.
 */
wkv7_status wkv7_decode_step(int32_t B, int32_t H, int32_t N, int32_t dtype, int32_t decay,
                             const void *r, const void *w, const void *k,
                             const void *v, const void *a, const void *b,
                             const float *s_in, float *s_out, void *y, void *stream);

/*
 * One decode step fused with the per-head output epilogue: the rwkv-lab page
 * ("RWKV community research additions") describes a one-token kernel that
 * carries the fp32 state update through GroupNorm, the RWKV bonus and output
 * gating, and the rwkv-metal page ("What's inside") names ln_x a GroupNorm per
 * head. Head size N = 64 only (other N: WKV7_ERR_UNSUPPORTED). The pages
 * print no formula; the reading taken, per (sequence, head h),
 * with y the plain step's output and mean / var the population mean and
 * variance of its N values:
 *   yn_i  = (y_i - mean(y)) / sqrt(var(y) + eps) * ln_w[h][i] + ln_b[h][i]
 *   out_i = (yn_i + (sum_j r_j k_j r_k[h][j]) * v_i) * g_i
 * Arguments as wkv7_decode_step, and:
 *   g          : [B,H,N] output gate (dtype); required.
 *   ln_w, ln_b : [H,N] fp32 GroupNorm affine; required.
 *   r_k        : [H,N] fp32 bonus weights; required.
 *   eps        : finite, >= 0 (else WKV7_ERR_INVALID_ARGUMENT).
 *   out        : [B,H,N] output (dtype); required.
 *   y          : [B,H,N] the plain step's y (dtype), or NULL to skip it.
 * The state is updated exactly as by wkv7_decode_step. All pointers 16-byte
 * aligned. Apart from s_out == s_in, no output (s_out, out, y) may share a
 * byte with an input (r..b, s_in, g, ln_w, ln_b, r_k) or another output.
 */
wkv7_status wkv7_decode_step_fused(int32_t B, int32_t H, int32_t N, int32_t dtype, int32_t decay,
                                   const void *r, const void *w, const void *k, const void *v,
                                   const void *a, const void *b, const float *s_in, float *s_out,
                                   const void *g, const float *ln_w, const float *ln_b,
                                   const float *r_k, float eps, void *out, void *y, void *stream);

/*
 * One token of a gated DeltaNet (GDN) layer, computed as one WKV-7 step (the
 * mapping of the rwkv-lab page, section "Highlight result -- GDN in
 * RWKV-7"). The gated delta rule
 *     S' = e^g S (I - beta k^ k^T) + beta v k^T,   out = S' q^ / sqrt(N)
 * equals S diag(e^g) + (S (-k^)) (beta e^g k^)^T + v (beta k^)^T: a WKV-7
 * step with decay e^g on every key, a = -k^, b = beta e^g k^ and write key
 * beta k^, read out with r = q^. Here q^ and k^ are the value head's key-head
 * q and k over max(||.||_2, 1e-12).
 *   N      : head size, 64 or 128 (GDN's matched geometry is 128; anything
 *            else: WKV7_ERR_UNSUPPORTED).
 *   H, Hk  : value heads and key heads, Hk divides H; value head h reads key
 *            head h / (H / Hk) (groups of consecutive value heads share one).
 *   q, k   : [B, Hk, N]; v, out : [B, H, N]; all of type dtype (fp32, bf16
 *            or fp16), 16-byte aligned. A q or k of length zero
 *            normalises to zero (the 1e-12 floor), so it stays finite: a
 *            zero k leaves the state only decayed, a zero q gives out = 0.
 *   g, beta: fp32 [B, H], 4-byte aligned: the log-decay and the write
 *            strength of each (sequence, value head).
 *   s_in, s_out : fp32 [B, H, N, N] (row = value index), 16-byte aligned;
 *            s_out == s_in updates in place. Any other overlap between an
 *            output (s_out, out) and an input or the other output is
 *            WKV7_ERR_INVALID_ARGUMENT.
 */
wkv7_status wkv7_gdn_decode_step(int32_t B, int32_t H, int32_t Hk, int32_t N, int32_t dtype,
                                 const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *s_in, float *s_out, void *out,
                                 void *stream);

/*
 * Workspace bytes of wkv7_gdn_forward: q^ and k^ in fp32, 2 * B*T*Hk*N * 4
 * (each part 256-byte aligned). N = 64 or 128 (else WKV7_ERR_UNSUPPORTED);
 * B, T, Hk >= 1 with B*T*Hk <= 2^24 (else WKV7_ERR_INVALID_ARGUMENT).
 */
wkv7_status wkv7_gdn_workspace_bytes(int32_t B, int32_t T, int32_t Hk, int32_t N, size_t *bytes);

/*
 * A dense batch of gated DeltaNet tokens (B rows of T tokens), each computed
 * as the WKV-7 step of wkv7_gdn_decode_step (rwkv-lab, "Highlight result --
 * GDN in RWKV-7"), token by token from s0 (or zero):
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T,
 *     out_t = S_t q^_t / sqrt(N),   x^ = x / max(||x||_2, 1e-12).
 *   q, k   : [B, T, Hk, N]; v, out : [B, T, H, N]; type dtype, 16-byte aligned.
 *   g, beta: fp32 [B, T, H], 4-byte aligned.
 *   s0     : fp32 [B, H, N, N] or NULL (zero initial state).
 *   s_out  : fp32 [B, H, N, N] final state, or NULL.
 *   workspace : >= wkv7_gdn_workspace_bytes(B, T, Hk, N), 16-byte aligned.
 * Value head h reads key head h / (H / Hk). H % Hk == 0 and B*H <= 2^24.
 * bf16 I/O evaluates the recurrence 16 tokens at a time in its chunk form
 * (products in three bf16 pieces, fp32 state); fp32 and fp16 token by token.
 * Outputs may not overlap inputs, each other or the workspace.
 */
wkv7_status wkv7_gdn_forward(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t N, int32_t dtype,
                             const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *s0, void *out, float *s_out,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace bytes of wkv7_gdn_backward: q^, k^ ([B,T,Hk,N] fp32 each), seven
 * remapped streams and six WKV-7 gradients ([B,T,H,N] fp32 each), the
 * checkpoints (B * ceil(T/16) x H x N x N fp32) and the WKV-7 backward's
 * workspace for fp32 streams at head size N, each part 256-byte aligned.
 * Sizes are checked as for wkv7_gdn_forward.
 */
wkv7_status wkv7_gdn_backward_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t N,
                                              size_t *bytes);

/*
 * Reverse-mode gradients of L = sum <dout, out> + <ds_out, S_T> for
 * wkv7_gdn_forward (rwkv-lab, "Highlight result -- GDN in RWKV-7"). That
 * forward is the WKV-7 step with decay exp(g) on every key, a-vector -k^,
 * b-vector beta exp(g) k^, written key k_w = beta k^ and read vector q^ (the
 * gated delta rule expanded); the gradients go back through it and through
 * the normalisation x^ = x / max(||x||_2, 1e-12):
 *     dk^ = beta dk_w - da + beta exp(g) db,  dq^ = dr (summed over the value
 *     heads of a key head);  dg = exp(g) (sum_j dw_j + beta sum_j db_j k^_j);
 *     dbeta = sum_j dk_w,j k^_j + exp(g) sum_j db_j k^_j;
 *     dx = (dx^ - x^ <x^, dx^>) / ||x|| (||x|| > 1e-12), dx^ / 1e-12 otherwise.
 *   q, k, v, g, beta, s0 : as for wkv7_gdn_forward.
 *   dout   : [B,T,H,N] (dtype) gradient of out, or NULL (zero).
 *   ds_out : fp32 [B,H,N,N] gradient of the final state, or NULL (zero).
 *   dq, dk : [B,T,Hk,N] (dtype); dv : [B,T,H,N] (dtype); dg, dbeta : fp32
 *            [B,T,H]; ds0 : fp32 [B,H,N,N] gradient of s0, or NULL.
 *   workspace : >= wkv7_gdn_backward_workspace_bytes(B, T, H, Hk, N),
 *            16-byte aligned, caller-owned; no two calls may share it at once.
 * The remapped streams are written in fp32, the WKV-7 forward (for its
 * checkpoints) and backward run on them at head size N, and two kernels
 * pull the gradients back. No output may overlap an input, another output
 * or the workspace: WKV7_ERR_INVALID_ARGUMENT, before any HIP call.
 */
wkv7_status wkv7_gdn_backward(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t N, int32_t dtype,
                              const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *s0, const void *dout, const float *ds_out,
                              void *dq, void *dk, void *dv, float *dg, float *dbeta, float *ds0,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Number of checkpoint slots a dense forward needs: B * ceil(T / 16). */
wkv7_status wkv7_checkpoint_slots(int32_t B, int32_t T, int64_t *slots);

/* Workspace bytes wkv7_backward needs for this descriptor. N = 64:
 * checkpoint slots (B * ceil(T / 16) dense, the segment table's slot count
 * otherwise) x H x (64 x 64 + 16 x 64 + 16 x 16) x 4; in segment mode plus
 * 4 x (1 + 2 x (ceil(slots / 8) + num_seqs)) bytes rounded up to 256 (room
 * for the list of (sequence, chunk group) work items of the second kernel).
 * N = 128: 0 (the backward needs no workspace). */
wkv7_status wkv7_workspace_bytes(const wkv7_desc *d, size_t *bytes);

/*
 * Host-side check of a segment table (host copies of seq_start / seq_len):
 * lengths >= 0, every sequence inside one row of T tokens, starts sorted and
 * sequences disjoint. Fills seq_ckpt_out[num_seqs] (may be NULL) with the
 * exclusive prefix sum of ceil(len / 16) and *slots_out (may be NULL) with
 * the total, i.e. the checkpoint layout wkv7_forward expects.
 */
wkv7_status wkv7_segments_check(int32_t B, int32_t T, int32_t num_seqs,
                                const int32_t *seq_start, const int32_t *seq_len,
                                int32_t *seq_ckpt_out, int64_t *slots_out);

const char *wkv7_status_string(wkv7_status s);
int32_t wkv7_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_H */
