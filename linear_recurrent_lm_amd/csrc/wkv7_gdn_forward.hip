// A sequence of gated DeltaNet (GDN) tokens through the RWKV-7 remap of the
// rwkv-lab page ("Highlight result -- GDN in RWKV-7"), at head size 128 (or
// 64). With q^ = q/||q||, k^ = k/||k|| and the remap r = q^, w = exp(g),
// k_write = beta k^, a = -k^, b = k^ exp(g) beta, the WKV-7 row update of
// value row i is
//     S_i <- exp(g) S_i + beta (v_i - exp(g) <S_i, k^>) k^,   out_i = <S_i, q^> / sqrt(N)
// (the gated delta rule, since the decay is one scalar per token and head).
//
// Two kernels. A pre-pass writes q^ and k^ in fp32 to the workspace (one
// wave per token row). The recurrence then runs token by token with one
// workgroup of N lanes per (sequence, value head): lane i holds state row i
// in N registers. The k^ and q^ rows of 16 tokens at a time are staged in
// LDS (double-buffered; the next block's loads fly while this block runs)
// and read by every lane as 16-byte broadcasts. Per token and lane: N
// multiply-adds for <S_i, k^>, 2N for the update, N for <S_i, q^>.
// Value head h reads key head h / (H / Hk).
#include "wkv7_kernels.h"

namespace wkv7 {
namespace {

template <typename TI, int N>
__global__ __launch_bounds__(256) void gdn_norm_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                       float *__restrict__ qn, float *__restrict__ kn,
                                                       int64_t rows) {
    constexpr int E = N / 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;               // whole waves leave together
    const int64_t o = row * N + lane * E;
    float a[E], b[E], sa = 0.f, sb = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        a[e] = IO<TI>::ld(q, o + e);
        b[e] = IO<TI>::ld(k, o + e);
        sa = fmaf(a[e], a[e], sa);
        sb = fmaf(b[e], b[e], sb);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        sa += __shfl_xor(sa, m);
        sb += __shfl_xor(sb, m);
    }
    const float ia = 1.f / sqrtf(sa), ib = 1.f / sqrtf(sb);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qn[o + e] = a[e] * ia;
        kn[o + e] = b[e] * ib;
    }
}

template <typename TI, int N>
__global__ __launch_bounds__(N) void gdn_fwd_kernel(int32_t T, int32_t H, int32_t Hk,
                                                   const float *__restrict__ qn, const float *__restrict__ kn,
                                                   const TI *__restrict__ v, const float *__restrict__ g,
                                                   const float *__restrict__ beta, const float *__restrict__ s0,
                                                   TI *__restrict__ out, float *__restrict__ s_out) {
    constexpr int TB = 16;                 // tokens per staged block
    constexpr int LD = TB * 2 * N / 4 / N; // float4 loads per thread per block (k^ and q^ rows)
    __shared__ __align__(16) float rows[2][TB][2][N];   // [buffer][token][k^, q^][N]
    const int64_t unit = blockIdx.x;       // b * H + h
    const int h = (int)(unit % H);
    const int64_t b = unit / H;
    const int kh = h / (H / Hk);
    const int i = threadIdx.x;
    const int64_t srow = (unit * N + i) * N;

    float S[N];
    if (s0) {
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            const f32x4 x = *(const f32x4 *)(s0 + srow + j);
            S[j] = x.x; S[j + 1] = x.y; S[j + 2] = x.z; S[j + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) S[j] = 0.f;
    }

    // Block loads: element c = q*N + i of the block's [TB][2][N/4] float4s
    // (token, k^ or q^, column quad); tokens past T are clamped to T-1.
    f32x4 st[LD];
    auto load_block = [&](int t0) {
#pragma unroll
        for (int q = 0; q < LD; ++q) {
            const int c = q * N + i;
            const int tt = c / (N / 2), which = (c / (N / 4)) & 1, quad = c % (N / 4);
            const int64_t tok = b * T + min(t0 + tt, T - 1);
            const float *src = which ? qn : kn;
            st[q] = *(const f32x4 *)(src + (tok * Hk + kh) * N + quad * 4);
        }
    };
    auto store_block = [&](int buf) {
#pragma unroll
        for (int q = 0; q < LD; ++q) {
            const int c = q * N + i;
            const int tt = c / (N / 2), which = (c / (N / 4)) & 1, quad = c % (N / 4);
            *(f32x4 *)&rows[buf][tt][which][quad * 4] = st[q];
        }
    };

    const float scale = 1.f / sqrtf((float)N);
    load_block(0);
    store_block(0);
    __syncthreads();
    const int nblk = (T + TB - 1) / TB;
    for (int blk = 0; blk < nblk; ++blk) {
        const int buf = blk & 1, t0 = blk * TB;
        if (blk + 1 < nblk) load_block(t0 + TB);
        const int tn = min(TB, T - t0);
        for (int tt = 0; tt < tn; ++tt) {
            const int64_t tok = b * T + t0 + tt;
            const float *kr = rows[buf][tt][0];
            const float *qr = rows[buf][tt][1];
            const float e = expf(g[tok * H + h]);
            const float bt = beta[tok * H + h];
            const float vi = IO<TI>::ld(v, (tok * H + h) * N + i);
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < N; j += 4) {
                const f32x4 kq = *(const f32x4 *)(kr + j);
                s4[0] = fmaf(S[j], kq.x, s4[0]);
                s4[1] = fmaf(S[j + 1], kq.y, s4[1]);
                s4[2] = fmaf(S[j + 2], kq.z, s4[2]);
                s4[3] = fmaf(S[j + 3], kq.w, s4[3]);
            }
            const float c = bt * fmaf(-e, (s4[0] + s4[1]) + (s4[2] + s4[3]), vi);
            float y4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < N; j += 4) {
                const f32x4 kq = *(const f32x4 *)(kr + j);
                const f32x4 qq = *(const f32x4 *)(qr + j);
                S[j] = fmaf(kq.x, c, S[j] * e);
                S[j + 1] = fmaf(kq.y, c, S[j + 1] * e);
                S[j + 2] = fmaf(kq.z, c, S[j + 2] * e);
                S[j + 3] = fmaf(kq.w, c, S[j + 3] * e);
                y4[0] = fmaf(S[j], qq.x, y4[0]);
                y4[1] = fmaf(S[j + 1], qq.y, y4[1]);
                y4[2] = fmaf(S[j + 2], qq.z, y4[2]);
                y4[3] = fmaf(S[j + 3], qq.w, y4[3]);
            }
            IO<TI>::st(out, (tok * H + h) * N + i, ((y4[0] + y4[1]) + (y4[2] + y4[3])) * scale);
        }
        if (blk + 1 < nblk) store_block(buf ^ 1);
        __syncthreads();
    }
    if (s_out) {
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            f32x4 x;
            x.x = S[j]; x.y = S[j + 1]; x.z = S[j + 2]; x.w = S[j + 3];
            *(f32x4 *)(s_out + srow + j) = x;
        }
    }
}

template <typename TI, int N>
hipError_t launch_typed_n(const GdnFwdArgs &a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.B * a.T * a.Hk;
    hipLaunchKernelGGL((gdn_norm_kernel<TI, N>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                       (const TI *)a.q, (const TI *)a.k, a.qn, a.kn, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_fwd_kernel<TI, N>), dim3((unsigned)((int64_t)a.B * a.H)), dim3(N), 0, stream,
                       a.T, a.H, a.Hk, (const float *)a.qn, (const float *)a.kn, (const TI *)a.v, a.g, a.beta,
                       a.s0, (TI *)a.out, a.s_out);
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_typed(const GdnFwdArgs &a, hipStream_t stream) {
    return a.N == 128 ? launch_typed_n<TI, 128>(a, stream) : launch_typed_n<TI, 64>(a, stream);
}

}  // namespace

hipError_t launch_gdn_forward(const GdnFwdArgs &a, hipStream_t stream) {
    if (a.dtype == 1) return launch_typed<uint16_t>(a, stream);
    if (a.dtype == 2) return launch_typed<_Float16>(a, stream);
    return launch_typed<float>(a, stream);
}

}  // namespace wkv7
