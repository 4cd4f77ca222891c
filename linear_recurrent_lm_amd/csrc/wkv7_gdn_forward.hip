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
// workgroup of N lanes per (sequence, value head). In wave v, lane l holds
// key half l / 32 of state rows 64 v + l % 32 and 64 v + l % 32 + 32, so every
// k^ or q^ value it reads serves two rows; the halves add their partial dot
// products with one lane exchange inside the wave. The k^ and q^ rows of 8
// tokens at a time are staged in LDS (double-buffered; the next block's loads
// fly while this block runs) and read as 16-byte broadcasts. Per token and
// row: N multiply-adds for <S_i, k^>, 2N for the update, N for <S_i, q^>.
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
    constexpr int TB = 8;                  // tokens per staged block
    constexpr int KH = N / 2;              // keys per lane
    constexpr int NQ = KH / 4;             // 16-byte quads per lane and row
    constexpr int LD = TB * 2 * N / 4 / N; // float4 loads per thread per block (k^ and q^ rows)
    __shared__ __align__(16) float rows[2][TB][2][N];   // [buffer][token][k^, q^][N], halves interleaved
    const int64_t unit = blockIdx.x;       // b * H + h
    const int h = (int)(unit % H);
    const int64_t b = unit / H;
    const int kh = h / (H / Hk);
    const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
    const int hf = ln >> 5;                           // key half: keys [hf KH, hf KH + KH)
    const int i0 = wv * 64 + (ln & 31), i1 = i0 + 32; // the lane's two state rows
    const int64_t srow0 = (unit * N + i0) * N + hf * KH;
    const int64_t srow1 = srow0 + 32 * N;

    float S0[KH], S1[KH];
    if (s0) {
#pragma unroll
        for (int j = 0; j < KH; j += 4) {
            const f32x4 x = *(const f32x4 *)(s0 + srow0 + j);
            S0[j] = x.x; S0[j + 1] = x.y; S0[j + 2] = x.z; S0[j + 3] = x.w;
            const f32x4 z = *(const f32x4 *)(s0 + srow1 + j);
            S1[j] = z.x; S1[j + 1] = z.y; S1[j + 2] = z.z; S1[j + 3] = z.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KH; ++j) S0[j] = S1[j] = 0.f;
    }

    // Block loads: element c = q*N + tid of the block's [TB][2][N/4] float4s
    // (token, k^ or q^, column quad); tokens past T are clamped to T-1. Quad
    // c4 of key half c4 / NQ is stored at slot 2 (c4 % NQ) + c4 / NQ, so the
    // two halves' broadcast reads fall in different banks.
    f32x4 st[LD];
    auto load_block = [&](int t0) {
#pragma unroll
        for (int q = 0; q < LD; ++q) {
            const int c = q * N + tid;
            const int tt = c / (N / 2), which = (c / (N / 4)) & 1, quad = c % (N / 4);
            const int64_t tok = b * T + min(t0 + tt, T - 1);
            const float *src = which ? qn : kn;
            st[q] = *(const f32x4 *)(src + (tok * Hk + kh) * N + quad * 4);
        }
    };
    auto store_block = [&](int buf) {
#pragma unroll
        for (int q = 0; q < LD; ++q) {
            const int c = q * N + tid;
            const int tt = c / (N / 2), which = (c / (N / 4)) & 1, quad = c % (N / 4);
            *(f32x4 *)&rows[buf][tt][which][4 * (2 * (quad % NQ) + quad / NQ)] = st[q];
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
            // the lane's key half: quad q of it at 8 q floats from here
            const float *kr = rows[buf][tt][0] + 4 * hf;
            const float *qr = rows[buf][tt][1] + 4 * hf;
            const float e = expf(g[tok * H + h]);
            const float bt = beta[tok * H + h];
            const float v0 = IO<TI>::ld(v, (tok * H + h) * N + i0);
            const float v1 = IO<TI>::ld(v, (tok * H + h) * N + i1);
            float p0[4] = {0.f, 0.f, 0.f, 0.f}, p1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 kq = *(const f32x4 *)(kr + 8 * q);
                const int j = 4 * q;
                p0[0] = fmaf(S0[j], kq.x, p0[0]);
                p0[1] = fmaf(S0[j + 1], kq.y, p0[1]);
                p0[2] = fmaf(S0[j + 2], kq.z, p0[2]);
                p0[3] = fmaf(S0[j + 3], kq.w, p0[3]);
                p1[0] = fmaf(S1[j], kq.x, p1[0]);
                p1[1] = fmaf(S1[j + 1], kq.y, p1[1]);
                p1[2] = fmaf(S1[j + 2], kq.z, p1[2]);
                p1[3] = fmaf(S1[j + 3], kq.w, p1[3]);
            }
            float sa0 = (p0[0] + p0[1]) + (p0[2] + p0[3]);
            float sa1 = (p1[0] + p1[1]) + (p1[2] + p1[3]);
            sa0 += __shfl_xor(sa0, 32);
            sa1 += __shfl_xor(sa1, 32);
            const float c0 = bt * fmaf(-e, sa0, v0);
            const float c1 = bt * fmaf(-e, sa1, v1);
            float y0[4] = {0.f, 0.f, 0.f, 0.f}, y1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 kq = *(const f32x4 *)(kr + 8 * q);
                const f32x4 qq = *(const f32x4 *)(qr + 8 * q);
                const int j = 4 * q;
                S0[j] = fmaf(kq.x, c0, S0[j] * e);
                S0[j + 1] = fmaf(kq.y, c0, S0[j + 1] * e);
                S0[j + 2] = fmaf(kq.z, c0, S0[j + 2] * e);
                S0[j + 3] = fmaf(kq.w, c0, S0[j + 3] * e);
                S1[j] = fmaf(kq.x, c1, S1[j] * e);
                S1[j + 1] = fmaf(kq.y, c1, S1[j + 1] * e);
                S1[j + 2] = fmaf(kq.z, c1, S1[j + 2] * e);
                S1[j + 3] = fmaf(kq.w, c1, S1[j + 3] * e);
                y0[0] = fmaf(S0[j], qq.x, y0[0]);
                y0[1] = fmaf(S0[j + 1], qq.y, y0[1]);
                y0[2] = fmaf(S0[j + 2], qq.z, y0[2]);
                y0[3] = fmaf(S0[j + 3], qq.w, y0[3]);
                y1[0] = fmaf(S1[j], qq.x, y1[0]);
                y1[1] = fmaf(S1[j + 1], qq.y, y1[1]);
                y1[2] = fmaf(S1[j + 2], qq.z, y1[2]);
                y1[3] = fmaf(S1[j + 3], qq.w, y1[3]);
            }
            float o0 = (y0[0] + y0[1]) + (y0[2] + y0[3]);
            float o1 = (y1[0] + y1[1]) + (y1[2] + y1[3]);
            o0 += __shfl_xor(o0, 32);
            o1 += __shfl_xor(o1, 32);
            // key half 0 writes row i0, key half 1 row i1: 64 consecutive outputs per wave
            IO<TI>::st(out, (tok * H + h) * N + (hf ? i1 : i0), (hf ? o1 : o0) * scale);
        }
        if (blk + 1 < nblk) store_block(buf ^ 1);
        __syncthreads();
    }
    if (s_out) {
#pragma unroll
        for (int j = 0; j < KH; j += 4) {
            *(f32x4 *)(s_out + srow0 + j) = f32x4{S0[j], S0[j + 1], S0[j + 2], S0[j + 3]};
            *(f32x4 *)(s_out + srow1 + j) = f32x4{S1[j], S1[j + 1], S1[j + 2], S1[j + 3]};
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
