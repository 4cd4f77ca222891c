// Launch interfaces of the WKV-7 kernels (host side, C++).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv7_device.h"

namespace wkv7 {

struct FwdArgs {
    SegParams seg;
    int dtype;                       // 0 fp32, 1 bf16, 2 fp16
    int logw;                        // 1: the w stream holds log(decay)
    const void *r, *w, *k, *v, *a, *b;
    const float *s0;
    void *y;
    float *s_out;
    float *ckpt;
};

struct BwdArgs {
    SegParams seg;
    int dtype;
    int logw;                        // 1: the w stream holds log(decay); dw is d/d log(decay)
    int grad_f32;                    // 1: dr..db are fp32
    const void *r, *w, *k, *v, *a, *b;
    const float *ckpt;
    const void *dy;
    const float *ds_out;
    void *dr, *dw, *dk, *dv, *da, *db;
    float *ds0;
    float *ws;                       // per-slot dS_C of the sweep ([slots][H][N][N] fp32, or the same array in
                                     // bf16 at the region's start for bf16 streams with bf16 gradients)
    float *ws_dr;                    // per-slot drhs = W^T dX of the sweep ([slots][H][16][N] fp32; bf16 likewise)
    float *ws_w;                     // per-slot W = (I - L_ab)^-1 of the sweep ([slots][H][16][16] fp32)
    // segment mode: the work items of the second pass, [count][(sequence,
    // chunk group) x glist_cap], written by a pre-pass into the workspace
    int32_t *glist;
    int64_t glist_cap;
    const void *staged[8];           // filled by the launcher: r w k a b v dy, null
};

struct DecArgs {
    int32_t B, H;
    int dtype;
    int logw;
    const void *r, *w, *k, *v, *a, *b;
    const float *s_in;
    float *s_out;
    void *y;                        // plain step: required; fused step: optional
    // fused output epilogue (out != nullptr): per-head GroupNorm of y with the
    // affine ln_w, ln_b ([H][N] fp32), plus the bonus (sum_j r_j k_j r_k[h][j]) v,
    // times the gate g ([B][H][N], I/O type)
    const void *g;
    const float *ln_w, *ln_b, *r_k;
    float eps;
    void *out;
};

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream);
// Backward, first pass: dS_C of every chunk into a.ws, and a.ds0.
hipError_t launch_backward_sweep(const BwdArgs &a, hipStream_t stream);
// Backward, second pass: per-chunk gradients from a.ckpt and a.ws.
hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);
// Head size 128: token-order backward of 8-row blocks; acc is a workspace of
// 5 x B*T*H*128 fp32 (the key-indexed gradients before their final dtype).
hipError_t launch_backward128(const BwdArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecArgs &a, hipStream_t stream);

// One token of a gated DeltaNet layer through the RWKV-7 remap.
struct GdnArgs {
    int32_t B, H, Hk, N;             // value heads H share Hk key heads; N = 64 or 128
    int dtype;
    const void *q, *k;               // [B][Hk][N], I/O type
    const void *v;                   // [B][H][N], I/O type
    const float *g, *beta;           // [B][H]
    const float *s_in;
    float *s_out;                    // [B][H][N][N]
    void *out;                       // [B][H][N], I/O type
};
hipError_t launch_gdn_decode(const GdnArgs &a, hipStream_t stream);
// The lean chunk-form forward (dense batches or segment tables; head size n
// = 64 or 128).
hipError_t launch_forward_cf(const FwdArgs &a, int n, hipStream_t stream);

// A sequence of GDN tokens through the remap (dense batch, no checkpoints).
struct GdnFwdArgs {
    int32_t B, T, H, Hk, N;
    int dtype;
    const void *q, *k;               // [B][T][Hk][N], I/O type
    const void *v;                   // [B][T][H][N], I/O type
    const float *g, *beta;           // [B][T][H]
    const float *s0;                 // [B][H][N][N] or null (zero)
    void *out;                       // [B][T][H][N], I/O type
    float *s_out;                    // [B][H][N][N] or null
    float *qn, *kn;                  // workspace: q^, k^ in fp32, [B][T][Hk][N] each
    float *ckpt;                     // chunk form only: [B * ceil(T / 16)][H][N][N], the state
                                     // entering each 16-token chunk, or null
};
hipError_t launch_gdn_forward(const GdnFwdArgs &a, hipStream_t stream);
// The recurrence of a bf16 GDN prefill in chunk form, after the q^, k^
// pre-pass (qn, kn filled).
hipError_t launch_gdn_forward_cf(const GdnFwdArgs &a, hipStream_t stream);
// q^, k^ of wkv7_gdn_forward's pre-pass, for `rows` token rows of N.
hipError_t launch_gdn_normalize(int dtype, int N, const void *q, const void *k, float *qn, float *kn,
                                int64_t rows, hipStream_t stream);
struct GdnBwdArgs {
    int32_t B, T, H, Hk, N;
    int dtype;
    const void *q, *k;               // [B][T][Hk][N], I/O type
    const void *v, *dout;            // [B][T][H][N], I/O type; dout may be null (zero)
    const float *g, *beta;           // [B][T][H]
    void *dq, *dk;                   // [B][T][Hk][N], I/O type
    void *dv;                        // [B][T][H][N], I/O type
    float *dg, *dbeta;               // [B][T][H]
    // fp32 workspace: q^, k^ [B][T][Hk][N]; the remapped WKV-7 streams and
    // dy = dout / sqrt(N), [B][T][H][N]; the WKV-7 gradients, [B][T][H][N]
    float *qn, *kn;
    float *r, *w, *kw, *v32, *a, *b, *dy;
    const float *gr, *gw, *gk, *gv, *ga, *gb;
};
hipError_t launch_gdn_remap(const GdnBwdArgs &a, hipStream_t stream);
hipError_t launch_gdn_pullback(const GdnBwdArgs &a, hipStream_t stream);
// The WKV-7 step (not fused) at head size 128.
hipError_t launch_decode128(const DecArgs &a, hipStream_t stream);

// Segment mode: write zeros to `nptr` token streams at tokens no sequence covers.
hipError_t launch_zero_uncovered(const SegParams &seg, int dtype, void *const *ptrs,
                                 int nptr, hipStream_t stream);

}  // namespace wkv7
