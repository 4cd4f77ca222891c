// WKV-7 forward, token order (RWKV-7 WKV-7 recurrence; the model card's
// "eager" token-order form). One wave per (sequence, head); lane i keeps state
// row S[i, :] in 64 VGPRs. Every 16 tokens the wave stages r, w, k, a, b, v of
// the chunk into LDS as fp32 (coalesced loads of each 64-element vector) and
// then walks the tokens: the key-indexed vectors are read back as LDS
// broadcasts, v_t[i] is per lane.
//
// Per token, lane i computes
//     sa   = sum_j S[i,j] a[j]                      (undecayed S_{t-1})
//     S[i,j] = S[i,j] w[j] + sa b[j] + v[i] k[j]
//     y[i] = sum_j S[i,j] r[j]                      (updated S_t)
// and the state entering tokens 0, 16, 32, ... of the sequence is stored as a
// checkpoint when requested.
#include "wkv7_kernels.h"

namespace wkv7 {
namespace {

constexpr int kStreams = 6;  // r, w, k, a, b, v in LDS

template <typename TI>
__global__ __launch_bounds__(64) void fwd_token_kernel(FwdArgs p) {
    const int H = p.seg.H;
    const int unit = blockIdx.x;
    const int h = unit % H;
    const int s = unit / H;
    const Unit u = resolve_unit(p.seg, s);
    const int i = threadIdx.x;

    const TI *__restrict__ r = (const TI *)p.r;
    const TI *__restrict__ w = (const TI *)p.w;
    const TI *__restrict__ k = (const TI *)p.k;
    const TI *__restrict__ v = (const TI *)p.v;
    const TI *__restrict__ a = (const TI *)p.a;
    const TI *__restrict__ b = (const TI *)p.b;
    TI *__restrict__ y = (TI *)p.y;

    __shared__ float tile[kChunk][kStreams][kN];

    float S[kN];
    const int64_t srow = ((int64_t)s * H + h) * kN * kN + (int64_t)i * kN;
    if (p.s0) {
#pragma unroll
        for (int j = 0; j < kN; j += 4) {
            const float4 q = *(const float4 *)(p.s0 + srow + j);
            S[j] = q.x; S[j + 1] = q.y; S[j + 2] = q.z; S[j + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kN; ++j) S[j] = 0.f;
    }

    const int64_t ts = (int64_t)H * kN;
    const int64_t base = (u.start * H + h) * kN;
#pragma unroll 1
    for (int t0 = 0; t0 < u.len; t0 += kChunk) {
        const int L = min(kChunk, u.len - t0);
        if (p.ckpt) {
            float *cp = p.ckpt + ((u.ckpt + t0 / kChunk) * H + h) * (int64_t)(kN * kN) + i * kN;
#pragma unroll
            for (int j = 0; j < kN; j += 4)
                *(float4 *)(cp + j) = make_float4(S[j], S[j + 1], S[j + 2], S[j + 3]);
        }
        __syncthreads();
        for (int t = 0; t < L; ++t) {
            const int64_t o = base + (int64_t)(t0 + t) * ts + i;
            tile[t][0][i] = IO<TI>::ld(r, o);
            tile[t][1][i] = IO<TI>::ld(w, o);
            tile[t][2][i] = IO<TI>::ld(k, o);
            tile[t][3][i] = IO<TI>::ld(a, o);
            tile[t][4][i] = IO<TI>::ld(b, o);
            tile[t][5][i] = IO<TI>::ld(v, o);
        }
        __syncthreads();
#pragma unroll 1
        for (int t = 0; t < L; ++t) {
            const float *rt = tile[t][0], *wt = tile[t][1], *kt = tile[t][2];
            const float *at = tile[t][3], *bt = tile[t][4];
            float s0a = 0.f, s1a = 0.f, s2a = 0.f, s3a = 0.f;
#pragma unroll
            for (int j = 0; j < kN; j += 4) {
                s0a = fmaf(S[j], at[j], s0a);
                s1a = fmaf(S[j + 1], at[j + 1], s1a);
                s2a = fmaf(S[j + 2], at[j + 2], s2a);
                s3a = fmaf(S[j + 3], at[j + 3], s3a);
            }
            const float sa = (s0a + s1a) + (s2a + s3a);
            const float vi = tile[t][5][i];
            float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
            for (int j = 0; j < kN; j += 4) {
                S[j] = fmaf(S[j], wt[j], fmaf(sa, bt[j], vi * kt[j]));
                S[j + 1] = fmaf(S[j + 1], wt[j + 1], fmaf(sa, bt[j + 1], vi * kt[j + 1]));
                S[j + 2] = fmaf(S[j + 2], wt[j + 2], fmaf(sa, bt[j + 2], vi * kt[j + 2]));
                S[j + 3] = fmaf(S[j + 3], wt[j + 3], fmaf(sa, bt[j + 3], vi * kt[j + 3]));
                y0 = fmaf(S[j], rt[j], y0);
                y1 = fmaf(S[j + 1], rt[j + 1], y1);
                y2 = fmaf(S[j + 2], rt[j + 2], y2);
                y3 = fmaf(S[j + 3], rt[j + 3], y3);
            }
            IO<TI>::st(y, base + (int64_t)(t0 + t) * ts + i, (y0 + y1) + (y2 + y3));
        }
    }
    if (p.s_out) {
#pragma unroll
        for (int j = 0; j < kN; j += 4)
            *(float4 *)(p.s_out + srow + j) = make_float4(S[j], S[j + 1], S[j + 2], S[j + 3]);
    }
}

}  // namespace

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream) {
    const int S = a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B;
    const dim3 grid((unsigned)((int64_t)S * a.seg.H));
    if (a.dtype == 1)
        hipLaunchKernelGGL(fwd_token_kernel<uint16_t>, grid, dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL(fwd_token_kernel<float>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace wkv7
