// Decode steps at head size 128 (and the GDN step at 64 too): one token per
// (sequence, head), fp32 state in and out, bound by HBM traffic (64 KiB of
// state in and 64 KiB out per (sequence, head) at N = 128).
//
// One 256-thread workgroup per (sequence, head): each state load instruction
// covers 4 KiB of contiguous memory (float4 index m*256 + tid), a lane owns
// 4 key columns of N*N/1024 rows, and the N/4 lanes that share a row reduce
// S a and S r (and, for GDN, the squared lengths of q and k) by lane
// exchange.
//
// The WKV-7 step (the rwkv-metal page's wkv7_step at the 128-wide heads the
// rwkv-lab conversion target uses) reads r, w, k, v, a, b as given:
//     S' = S diag(w) + (S a) b^T + v k^T,   y = S' r.
//
// The gated DeltaNet (GDN) step runs as one WKV-7 step, the mapping of the
// rwkv-lab page ("Highlight result -- GDN in RWKV-7"). The gated delta rule
//     S' = e^g S (I - beta k^ k^T) + beta v k^T
// expands to S diag(e^g) + (S (-k^)) (beta e^g k^)^T + v (beta k^)^T: a WKV-7
// step whose decay is e^g on every key, whose a and b are -k^ and beta e^g k^,
// and whose write key is beta k^. Reading it out with r = q^ and scaling by
// 1/sqrt(N) gives GDN's output. Here q^ and k^ are q and k over
// max(||.||_2, 1e-12).
// Value head h reads key head h / (H / Hk): groups of consecutive value heads
// share a key head (GDN's geometry is 32 value heads over 16 key heads).
#include "wkv7_kernels.h"

namespace wkv7 {
namespace {

template <int L>
__device__ __forceinline__ float sum_lanes(float x) {
#pragma unroll
    for (int o = 1; o < L; o <<= 1) x += __shfl_xor(x, o, L);
    return x;
}

template <typename TI, int N>
__global__ __launch_bounds__(256) void gdn_decode_kernel(GdnArgs p) {
    constexpr int LPR = N / 4;           // lanes per state row
    constexpr int RPI = 256 / LPR;       // rows per load instruction of the workgroup
    constexpr int IT = N / RPI;          // load instructions per workgroup
    const int64_t unit = blockIdx.x;     // b * H + h
    const int h = (int)(unit % p.H);
    const int64_t bq = unit / p.H;
    const int kh = h / (p.H / p.Hk);
    const int tid = threadIdx.x;
    const int c0 = (tid % LPR) * 4;
    const int rl = tid / LPR;
    const int64_t sb = unit * (int64_t)(N * N);
    const int64_t vb = unit * N;
    const int64_t kb = (bq * p.Hk + kh) * N;

    f32x4 S[IT];
#pragma unroll
    for (int m = 0; m < IT; ++m)
        S[m] = __builtin_nontemporal_load((const f32x4 *)(p.s_in + sb) + m * 256 + tid);

    float q[4], k[4], vv[IT];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        q[e] = IO<TI>::ld((const TI *)p.q, kb + c0 + e);
        k[e] = IO<TI>::ld((const TI *)p.k, kb + c0 + e);
    }
#pragma unroll
    for (int m = 0; m < IT; ++m) vv[m] = IO<TI>::ld((const TI *)p.v, vb + m * RPI + rl);
    // x / max(||x||, 1e-12): a zero q or k normalises to zero, not NaN
    const float qs = 1.f / fmaxf(sqrtf(sum_lanes<LPR>(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3])),
                                 kGdnNormEps);
    const float ks = 1.f / fmaxf(sqrtf(sum_lanes<LPR>(k[0] * k[0] + k[1] * k[1] + k[2] * k[2] + k[3] * k[3])),
                                 kGdnNormEps);
    const float decay = expf(p.g[unit]);
    const float beta = p.beta[unit];
    float r[4], a[4], b[4], kw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float kn = k[e] * ks;
        r[e] = q[e] * qs;
        a[e] = -kn;
        b[e] = kn * decay * beta;
        kw[e] = beta * kn;
    }

    const float scale = 1.f / sqrtf((float)N);
    float yv[IT];
#pragma unroll
    for (int m = 0; m < IT; ++m) {
        const float sa = sum_lanes<LPR>(S[m].x * a[0] + S[m].y * a[1] + S[m].z * a[2] + S[m].w * a[3]);
        const float vi = vv[m];
        S[m].x = fmaf(S[m].x, decay, fmaf(sa, b[0], vi * kw[0]));
        S[m].y = fmaf(S[m].y, decay, fmaf(sa, b[1], vi * kw[1]));
        S[m].z = fmaf(S[m].z, decay, fmaf(sa, b[2], vi * kw[2]));
        S[m].w = fmaf(S[m].w, decay, fmaf(sa, b[3], vi * kw[3]));
        yv[m] = sum_lanes<LPR>(S[m].x * r[0] + S[m].y * r[1] + S[m].z * r[2] + S[m].w * r[3]) * scale;
    }
#pragma unroll
    for (int m = 0; m < IT; ++m)
        __builtin_nontemporal_store(S[m], (f32x4 *)(p.s_out + sb) + m * 256 + tid);
    if (tid % LPR == 0) {
#pragma unroll
        for (int m = 0; m < IT; ++m) IO<TI>::st((TI *)p.out, vb + m * RPI + rl, yv[m]);
    }
}

// The WKV-7 step at N = 128 (same layout as above).
template <typename TI>
__global__ __launch_bounds__(256) void decode128_kernel(DecArgs p) {
    constexpr int N = 128, LPR = 32, RPI = 8, IT = 16;
    const int64_t unit = blockIdx.x;
    const int tid = threadIdx.x;
    const int c0 = (tid % LPR) * 4;
    const int rl = tid / LPR;
    const int64_t sb = unit * (int64_t)(N * N);
    const int64_t vb = unit * N;

    f32x4 S[IT];
#pragma unroll
    for (int m = 0; m < IT; ++m)
        S[m] = __builtin_nontemporal_load((const f32x4 *)(p.s_in + sb) + m * 256 + tid);
    float r[4], w[4], k[4], a[4], b[4], vv[IT];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = IO<TI>::ld((const TI *)p.r, vb + c0 + e);
        w[e] = IO<TI>::ld((const TI *)p.w, vb + c0 + e);
        k[e] = IO<TI>::ld((const TI *)p.k, vb + c0 + e);
        a[e] = IO<TI>::ld((const TI *)p.a, vb + c0 + e);
        b[e] = IO<TI>::ld((const TI *)p.b, vb + c0 + e);
    }
    decay_of<4>(w, p.logw);
#pragma unroll
    for (int m = 0; m < IT; ++m) vv[m] = IO<TI>::ld((const TI *)p.v, vb + m * RPI + rl);

    float yv[IT];
#pragma unroll
    for (int m = 0; m < IT; ++m) {
        const float sa = sum_lanes<LPR>(S[m].x * a[0] + S[m].y * a[1] + S[m].z * a[2] + S[m].w * a[3]);
        const float vi = vv[m];
        S[m].x = fmaf(S[m].x, w[0], fmaf(sa, b[0], vi * k[0]));
        S[m].y = fmaf(S[m].y, w[1], fmaf(sa, b[1], vi * k[1]));
        S[m].z = fmaf(S[m].z, w[2], fmaf(sa, b[2], vi * k[2]));
        S[m].w = fmaf(S[m].w, w[3], fmaf(sa, b[3], vi * k[3]));
        yv[m] = sum_lanes<LPR>(S[m].x * r[0] + S[m].y * r[1] + S[m].z * r[2] + S[m].w * r[3]);
    }
#pragma unroll
    for (int m = 0; m < IT; ++m)
        __builtin_nontemporal_store(S[m], (f32x4 *)(p.s_out + sb) + m * 256 + tid);
    if (tid % LPR == 0) {
#pragma unroll
        for (int m = 0; m < IT; ++m) IO<TI>::st((TI *)p.y, vb + m * RPI + rl, yv[m]);
    }
}

template <int N>
hipError_t launch_n(const GdnArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.B * a.H));
    if (a.dtype == 1) hipLaunchKernelGGL((gdn_decode_kernel<uint16_t, N>), grid, dim3(256), 0, stream, a);
    else if (a.dtype == 2) hipLaunchKernelGGL((gdn_decode_kernel<_Float16, N>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((gdn_decode_kernel<float, N>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_decode(const GdnArgs &a, hipStream_t stream) {
    return a.N == 128 ? launch_n<128>(a, stream) : launch_n<64>(a, stream);
}

hipError_t launch_decode128(const DecArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.B * a.H));
    if (a.dtype == 1) hipLaunchKernelGGL(decode128_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
    else if (a.dtype == 2) hipLaunchKernelGGL(decode128_kernel<_Float16>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(decode128_kernel<float>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace wkv7
