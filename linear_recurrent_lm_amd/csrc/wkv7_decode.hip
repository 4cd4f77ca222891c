// WKV-7 decode step: one token for each (sequence, head), state read and
// written in fp32 (the rwkv-metal page's wkv7_step; the rwkv-lab page's
// in-place one-token state transition). The step is bound by HBM traffic:
// 16 KiB of state in and 16 KiB out per (sequence, head) against 9 flop per
// state element.
//
// One 256-thread workgroup per (sequence, head). The 64x64 state is read as
// 1024 float4 with float4 index m*256 + tid (m = 0..3), so each load
// instruction of the workgroup covers 4 KiB of contiguous memory. Thread tid
// then owns rows m*16 + tid/16 and columns 4*(tid%16) .. +3; the row sums
// S a and S r reduce over the 16 lanes sharing a row (one DPP row).
//
// The fused variant carries y through the per-head output epilogue (the
// rwkv-lab page, "RWKV community research additions": one kernel for the
// state update, GroupNorm, the RWKV bonus and output gating; the rwkv-metal
// page, "What's inside": ln_x is a GroupNorm per head):
//     yn_i  = (y_i - mean(y)) / sqrt(var(y) + eps) * ln_w[h][i] + ln_b[h][i]
//     out_i = (yn_i + (sum_j r_j k_j r_k[h][j]) v_i) * g_i
// with the population mean and variance of the head's 64 values, formed in
// two passes (sums over a wave's rows by lane exchange, then over the four
// waves through LDS). The bonus sum runs over the key columns, which every
// 16-lane row group already spans.
#include "wkv7_kernels.h"

namespace wkv7 {
namespace {

__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 8, 16);
    return x;
}

template <typename TI>
__device__ __forceinline__ void ld4(const TI *p, int64_t o, float *x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = IO<TI>::ld(p, o + e);
}

template <typename TI, bool FUSED>
__global__ __launch_bounds__(256) void decode_kernel(DecArgs p) {
    const int64_t unit = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t sb = unit * (kN * kN);
    const int64_t vb = unit * kN;
    const int c0 = (tid & 15) * 4;
    const int rl = tid >> 4;

    f32x4 S[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        S[m] = __builtin_nontemporal_load((const f32x4 *)(p.s_in + sb) + m * 256 + tid);

    float a[4], w[4], b[4], k[4], r[4], vv[4];
    ld4((const TI *)p.a, vb + c0, a);
    ld4((const TI *)p.w, vb + c0, w);
    decay_of<4>(w, p.logw);
    ld4((const TI *)p.b, vb + c0, b);
    ld4((const TI *)p.k, vb + c0, k);
    ld4((const TI *)p.r, vb + c0, r);
#pragma unroll
    for (int m = 0; m < 4; ++m) vv[m] = IO<TI>::ld((const TI *)p.v, vb + m * 16 + rl);

    float yv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float sa = S[m].x * a[0] + S[m].y * a[1] + S[m].z * a[2] + S[m].w * a[3];
        sa = sum16(sa);
        const float vi = vv[m];
        S[m].x = fmaf(S[m].x, w[0], fmaf(sa, b[0], vi * k[0]));
        S[m].y = fmaf(S[m].y, w[1], fmaf(sa, b[1], vi * k[1]));
        S[m].z = fmaf(S[m].z, w[2], fmaf(sa, b[2], vi * k[2]));
        S[m].w = fmaf(S[m].w, w[3], fmaf(sa, b[3], vi * k[3]));
        yv[m] = sum16(S[m].x * r[0] + S[m].y * r[1] + S[m].z * r[2] + S[m].w * r[3]);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
        __builtin_nontemporal_store(S[m], (f32x4 *)(p.s_out + sb) + m * 256 + tid);
    if (!FUSED || p.y) {
        if ((tid & 15) == 0) {
#pragma unroll
            for (int m = 0; m < 4; ++m) IO<TI>::st((TI *)p.y, vb + m * 16 + rl, yv[m]);
        }
    }
    if constexpr (FUSED) {
        __shared__ float red[8];
        const int h = (int)(unit % p.H), wq = tid >> 6;
        // a wave's 16 rows: its 4 row groups (lanes l, l^16, l^32, l^48) x 4 rows
        float ps = (yv[0] + yv[1]) + (yv[2] + yv[3]);
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        if ((tid & 63) == 0) red[wq] = ps;
        __syncthreads();
        const float mean = ((red[0] + red[1]) + (red[2] + red[3])) * (1.f / kN);
        float d[4], pq = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            d[m] = yv[m] - mean;
            pq = fmaf(d[m], d[m], pq);
        }
        pq += __shfl_xor(pq, 16);
        pq += __shfl_xor(pq, 32);
        if ((tid & 63) == 0) red[4 + wq] = pq;
        __syncthreads();
        const float var = ((red[4] + red[5]) + (red[6] + red[7])) * (1.f / kN);
        const float inv = 1.f / sqrtf(var + p.eps);
        const float *rk = p.r_k + (int64_t)h * kN + c0;
        float bz = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) bz = fmaf(r[e] * k[e], rk[e], bz);
        bz = sum16(bz);
        if ((tid & 15) == 0) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int i = m * 16 + rl;
                const float yn = fmaf(d[m] * inv, p.ln_w[(int64_t)h * kN + i], p.ln_b[(int64_t)h * kN + i]);
                const float gi = IO<TI>::ld((const TI *)p.g, vb + i);
                IO<TI>::st((TI *)p.out, vb + i, fmaf(bz, vv[m], yn) * gi);
            }
        }
    }
}

}  // namespace

hipError_t launch_decode(const DecArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.B * a.H));
    const bool fused = a.out != nullptr;
    if (a.dtype == 1) {
        if (fused) hipLaunchKernelGGL((decode_kernel<uint16_t, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<uint16_t, false>), grid, dim3(256), 0, stream, a);
    } else if (a.dtype == 2) {
        if (fused) hipLaunchKernelGGL((decode_kernel<_Float16, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<_Float16, false>), grid, dim3(256), 0, stream, a);
    } else {
        if (fused) hipLaunchKernelGGL((decode_kernel<float, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<float, false>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace wkv7
