// Gated DeltaNet (GDN) backward, through the WKV-7 form of the gated delta
// rule that the rwkv-lab page's section "Highlight result -- GDN in RWKV-7"
// proposes. The rule S' = e^g S (I - beta k^ k^T) + beta v k^T is the WKV-7
// step with decay e^g on every key, a-vector -k^, b-vector beta e^g k^ and
// written key beta k^; the output reads along q^ and is scaled by 1/sqrt(N)
// (x^ = x / max(||x||_2, 1e-12); value head h reads key head h / (H / Hk)).
// The backward writes those five vectors, v and dy = dout / sqrt(N) as fp32
// streams, runs the WKV-7 forward (for the checkpoints) and backward on them,
// and applies the chain rule to the WKV-7 gradients:
//     the key's total dk^ = beta dk_w - da + beta e^g db, and dq^ = dr, each
//         summed over the value heads of a key head;
//     dg = e^g (sum_j dw_j + beta sum_j db_j k^_j)   (every key's decay is e^g);
//     dbeta = sum_j dk_w,j k^_j + e^g sum_j db_j k^_j;
//     through the normalisation dx = (dx^ - x^ <x^, dx^>) / ||x|| when
//         ||x|| > 1e-12, and dx^ / 1e-12 otherwise.
// This file holds the remap and the pull-back; the WKV-7 calls are the
// library's own.
#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

// sum over the 64 lanes of a wave, in every lane
__device__ __forceinline__ float wave_sum(float x) {
    float a = sum16(x), b = a;
    swap16(a, b);                 // even rows: rows 0 and 1 (2 and 3) of the half
    float c = a + b, d = c;
    swap32(c, d);                 // both halves
    return c + d;
}

template <typename TI>
__device__ __forceinline__ float4 ld4(const TI *p, int64_t i) {
    return make_float4(IO<TI>::ld(p, i), IO<TI>::ld(p, i + 1), IO<TI>::ld(p, i + 2), IO<TI>::ld(p, i + 3));
}

// The remapped WKV-7 streams, 4 elements per thread.
template <typename TI>
__global__ __launch_bounds__(256) void gdn_remap_kernel(GdnBwdArgs p) {
    const int64_t n4 = (int64_t)p.B * p.T * p.H * p.N / 4;
    const int grp = p.H / p.Hk;
    const float inv_sqrt_n = 1.f / sqrtf((float)p.N);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = 4 * i;
        const int64_t row = e / p.N;                  // (b T + t) H + h
        const int j = (int)(e - row * p.N);
        const int h = (int)(row % p.H);
        const int64_t krow = (row / p.H) * p.Hk + h / grp;
        const float4 qn = *(const float4 *)(p.qn + krow * p.N + j);
        const float4 kn = *(const float4 *)(p.kn + krow * p.N + j);
        const float eg = expf(p.g[row]), bt = p.beta[row], be = bt * eg;
        *(float4 *)(p.r + e) = qn;
        *(float4 *)(p.w + e) = make_float4(eg, eg, eg, eg);
        *(float4 *)(p.kw + e) = make_float4(bt * kn.x, bt * kn.y, bt * kn.z, bt * kn.w);
        *(float4 *)(p.a + e) = make_float4(-kn.x, -kn.y, -kn.z, -kn.w);
        *(float4 *)(p.b + e) = make_float4(be * kn.x, be * kn.y, be * kn.z, be * kn.w);
        *(float4 *)(p.v32 + e) = ld4((const TI *)p.v, e);
        if (p.dout) {
            const float4 d = ld4((const TI *)p.dout, e);
            *(float4 *)(p.dy + e) = make_float4(d.x * inv_sqrt_n, d.y * inv_sqrt_n, d.z * inv_sqrt_n, d.w * inv_sqrt_n);
        }
    }
}

// Per value-head row (one wave): dg, dbeta and dv.
template <typename TI, int N>
__global__ __launch_bounds__(256) void gdn_pull_value_kernel(GdnBwdArgs p, int64_t rows) {
    constexpr int E = N / 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;                          // whole waves leave together
    const int grp = p.H / p.Hk;
    const int64_t krow = (row / p.H) * p.Hk + (row % p.H) / grp;
    float sw = 0.f, sb = 0.f, sk = 0.f;
#pragma unroll
    for (int q = 0; q < E; ++q) {
        const int64_t o = row * N + lane * E + q;
        const float kn = p.kn[krow * N + lane * E + q];
        sw += p.gw[o];
        sb = fmaf(p.gb[o], kn, sb);
        sk = fmaf(p.gk[o], kn, sk);
        IO<TI>::st((TI *)p.dv, o, p.gv[o]);
    }
    sw = wave_sum(sw);
    sb = wave_sum(sb);
    sk = wave_sum(sk);
    if (lane == 0) {
        const float eg = expf(p.g[row]);
        p.dg[row] = eg * fmaf(p.beta[row], sb, sw);
        p.dbeta[row] = fmaf(eg, sb, sk);
    }
}

// Per key-head row (one wave): dq^, dk^ summed over the value heads of the
// key head, then through the normalisation.
template <typename TI, int N>
__global__ __launch_bounds__(256) void gdn_pull_key_kernel(GdnBwdArgs p, int64_t rows) {
    constexpr int E = N / 64;
    const int64_t krow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (krow >= rows) return;
    const int grp = p.H / p.Hk;
    const int64_t bt = krow / p.Hk;                   // b T + t
    const int kh = (int)(krow % p.Hk);
    float dqn[E], dkn[E], qn[E], kn[E], q[E], k[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t o = krow * N + lane * E + e;
        dqn[e] = dkn[e] = 0.f;
        qn[e] = p.qn[o];
        kn[e] = p.kn[o];
        q[e] = IO<TI>::ld((const TI *)p.q, o);
        k[e] = IO<TI>::ld((const TI *)p.k, o);
    }
    for (int hh = 0; hh < grp; ++hh) {
        const int64_t row = bt * p.H + kh * grp + hh;
        const float bet = p.beta[row], be = bet * expf(p.g[row]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int64_t o = row * N + lane * E + e;
            dqn[e] += p.gr[o];
            dkn[e] += fmaf(bet, p.gk[o], fmaf(be, p.gb[o], -p.ga[o]));
        }
    }
    float sq = 0.f, sk = 0.f, pq = 0.f, pk = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        sq = fmaf(q[e], q[e], sq);
        sk = fmaf(k[e], k[e], sk);
        pq = fmaf(qn[e], dqn[e], pq);
        pk = fmaf(kn[e], dkn[e], pk);
    }
    const float nq = sqrtf(wave_sum(sq)), nk = sqrtf(wave_sum(sk));
    pq = wave_sum(pq);
    pk = wave_sum(pk);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t o = krow * N + lane * E + e;
        const float dq = nq > kGdnNormEps ? (dqn[e] - qn[e] * pq) / nq : dqn[e] / kGdnNormEps;
        const float dk = nk > kGdnNormEps ? (dkn[e] - kn[e] * pk) / nk : dkn[e] / kGdnNormEps;
        IO<TI>::st((TI *)p.dq, o, dq);
        IO<TI>::st((TI *)p.dk, o, dk);
    }
}

template <typename TI>
hipError_t remap_t(const GdnBwdArgs &a, hipStream_t stream) {
    const int64_t n4 = (int64_t)a.B * a.T * a.H * a.N / 4;
    const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 8192);
    hipLaunchKernelGGL(gdn_remap_kernel<TI>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename TI, int N>
hipError_t pull_t(const GdnBwdArgs &a, hipStream_t stream) {
    const int64_t vrows = (int64_t)a.B * a.T * a.H, krows = (int64_t)a.B * a.T * a.Hk;
    hipLaunchKernelGGL((gdn_pull_value_kernel<TI, N>), dim3((unsigned)((vrows + 3) / 4)), dim3(256), 0, stream, a,
                       vrows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_pull_key_kernel<TI, N>), dim3((unsigned)((krows + 3) / 4)), dim3(256), 0, stream, a,
                       krows);
    return hipGetLastError();
}

template <typename TI>
hipError_t pull_ti(const GdnBwdArgs &a, hipStream_t stream) {
    return a.N == 128 ? pull_t<TI, 128>(a, stream) : pull_t<TI, 64>(a, stream);
}

}  // namespace

hipError_t launch_gdn_remap(const GdnBwdArgs &a, hipStream_t stream) {
    hipError_t e = launch_gdn_normalize(a.dtype, a.N, a.q, a.k, a.qn, a.kn, (int64_t)a.B * a.T * a.Hk, stream);
    if (e != hipSuccess) return e;
    if (a.dtype == 1) return remap_t<uint16_t>(a, stream);
    if (a.dtype == 2) return remap_t<_Float16>(a, stream);
    return remap_t<float>(a, stream);
}

hipError_t launch_gdn_pullback(const GdnBwdArgs &a, hipStream_t stream) {
    if (a.dtype == 1) return pull_ti<uint16_t>(a, stream);
    if (a.dtype == 2) return pull_ti<_Float16>(a, stream);
    return pull_ti<float>(a, stream);
}

}  // namespace wkv7
