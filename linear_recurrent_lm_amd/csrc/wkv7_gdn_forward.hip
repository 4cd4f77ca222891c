// A sequence of gated DeltaNet (GDN) tokens, run as WKV-7 steps as the
// rwkv-lab page's section "Highlight result -- GDN in RWKV-7" proposes, at
// head size 128 (or 64). Expanding the gated delta rule
//     S' = e^g S (I - beta k^ k^T) + beta v k^T
// gives S' = S diag(e^g) + (S a) b^T + v k_w^T with the decay e^g on every
// key, a = -k^ and b = beta e^g k^ (the sign could sit on either), and the
// written key k_w = beta k^; the output reads S' along q^ and is scaled by
// 1/sqrt(N). For value row i:
//     S_i <- exp(g) S_i + beta (v_i - exp(g) <S_i, k^>) k^,   out_i = <S_i, q^> / sqrt(N)
// (q^, k^: q and k over max(||.||_2, 1e-12), so a zero row gives a zero vector).
//
// Two kernels. A pre-pass writes q^ and k^ in fp32 to the workspace (one
// wave per token row). The recurrence then runs token by token with one
// workgroup of 2N lanes per (sequence, value head). In wave v, lane l holds
// key half l / 32 of state row 32 v + l % 32; the halves add their partial
// dot products with one register swap between the wave's halves. (Two rows
// per lane on N lanes ran one wave per SIMD at the prefill shape; one row on
// 2N lanes runs two.) The k^ and q^ rows of 8 tokens at a time are staged in
// LDS (double-buffered; the next block's loads fly while this block runs) and
// read as 16-byte broadcasts. Per token and row: N multiply-adds for
// <S_i, k^>, 2N for the update, N for <S_i, q^>.
// Value head h reads key head h / (H / Hk).
#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

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
    // x / max(||x||, 1e-12): a zero row normalises to zero, not NaN
    const float ia = 1.f / fmaxf(sqrtf(sa), kGdnNormEps), ib = 1.f / fmaxf(sqrtf(sb), kGdnNormEps);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qn[o + e] = a[e] * ia;
        kn[o + e] = b[e] * ib;
    }
}

template <typename TI, int N>
__global__ __launch_bounds__(2 * N) void gdn_fwd_kernel(int32_t T, int32_t H, int32_t Hk,
                                                   const float *__restrict__ qn, const float *__restrict__ kn,
                                                   const TI *__restrict__ v, const float *__restrict__ g,
                                                   const float *__restrict__ beta, const float *__restrict__ s0,
                                                   TI *__restrict__ out, float *__restrict__ s_out) {
    constexpr int NT = 2 * N;              // threads: one state row per lane
    constexpr int TB = 8;                  // tokens per staged block
    constexpr int KH = N / 2;              // keys per lane
    constexpr int NQ = KH / 4;             // 16-byte quads per lane and row
    constexpr int LD = TB * 2 * N / 4 / NT; // float4 loads per thread per block (k^ and q^ rows)
    static_assert(TB * 2 * N / 4 % NT == 0, "whole loads per thread");
    __shared__ __align__(16) float rows[2][TB][2][N];   // [buffer][token][k^, q^][N], halves interleaved
    const int64_t unit = blockIdx.x;       // b * H + h
    const int h = (int)(unit % H);
    const int64_t b = unit / H;
    const int kh = h / (H / Hk);
    const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
    const int hf = ln >> 5;                           // key half: keys [hf KH, hf KH + KH)
    const int i0 = wv * 32 + (ln & 31);               // the lane's state row
    const int64_t srow0 = (unit * N + i0) * N + hf * KH;

    float S0[KH];
    if (s0) {
#pragma unroll
        for (int j = 0; j < KH; j += 4) {
            const f32x4 x = *(const f32x4 *)(s0 + srow0 + j);
            S0[j] = x.x; S0[j + 1] = x.y; S0[j + 2] = x.z; S0[j + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KH; ++j) S0[j] = 0.f;
    }

    // Block loads: element c = q*NT + tid of the block's [TB][2][N/4] float4s
    // (token, k^ or q^, column quad); tokens past T are clamped to T-1. Quad
    // c4 of key half c4 / NQ is stored at slot 2 (c4 % NQ) + c4 / NQ, so the
    // two halves' broadcast reads fall in different banks.
    f32x4 st[LD];
    auto load_block = [&](int t0) {
#pragma unroll
        for (int q = 0; q < LD; ++q) {
            const int c = q * NT + tid;
            const int tt = c / (N / 2), which = (c / (N / 4)) & 1, quad = c % (N / 4);
            const int64_t tok = b * T + min(t0 + tt, T - 1);
            const float *src = which ? qn : kn;
            st[q] = *(const f32x4 *)(src + (tok * Hk + kh) * N + quad * 4);
        }
    };
    auto store_block = [&](int buf) {
#pragma unroll
        for (int q = 0; q < LD; ++q) {
            const int c = q * NT + tid;
            const int tt = c / (N / 2), which = (c / (N / 4)) & 1, quad = c % (N / 4);
            *(f32x4 *)&rows[buf][tt][which][4 * (2 * (quad % NQ) + quad / NQ)] = st[q];
        }
    };
    // the sum of the row's two key halves (lanes l and l ^ 32), in both
    auto halves = [](float x) {
        float lo = x, hi = x;
        swap32(lo, hi);
        return lo + hi;
    };

    // The state is kept as S = G Sh, G the running product of the decays
    // since the last fold: the decay then leaves the per-element update,
    //     Sh_i <- Sh_i + (c_i / G') k^,   c_i = beta (v_i - G' <Sh_i, k^>),
    //     out_i = G' <Sh_i, q^> / sqrt(N),  G' = G exp(g),
    // which is the gated delta rule for S_i. When G' would fall below 2^-60
    // (or exp(g) is 0), G' is first folded into Sh (Sh <- G' Sh, G' = 1),
    // which leaves the same formula exact, so 1 / G' stays below 2^60 and
    // every term is an fp32 number.
    constexpr float kFoldBelow = 0x1p-60f;
    float G = 1.f;
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
            float Gn = G * e;
            if (!(Gn >= kFoldBelow)) {                           // uniform: g is per (token, head)
                // fold the running product and this token's decay into Sh
#pragma unroll
                for (int j = 0; j < KH; ++j) S0[j] *= Gn;
                Gn = 1.f;
            }
            const float btg = bt / Gn;                         // off the dot product's path
            float p0[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 kq = *(const f32x4 *)(kr + 8 * q);
                const int j = 4 * q;
                p0[0] = fmaf(S0[j], kq.x, p0[0]);
                p0[1] = fmaf(S0[j + 1], kq.y, p0[1]);
                p0[2] = fmaf(S0[j + 2], kq.z, p0[2]);
                p0[3] = fmaf(S0[j + 3], kq.w, p0[3]);
            }
            const float sk = halves((p0[0] + p0[1]) + (p0[2] + p0[3]));   // <Sh, k^>
            // S_{t-1} = G Sh, so e <S_{t-1}, k^> = Gn <Sh, k^> (after a fold Sh
            // already holds e S_{t-1} and Gn is 1)
            const float ci = btg * fmaf(-Gn, sk, v0);
            float y0[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 kq = *(const f32x4 *)(kr + 8 * q);
                const f32x4 qq = *(const f32x4 *)(qr + 8 * q);
                const int j = 4 * q;
                S0[j] = fmaf(kq.x, ci, S0[j]);
                S0[j + 1] = fmaf(kq.y, ci, S0[j + 1]);
                S0[j + 2] = fmaf(kq.z, ci, S0[j + 2]);
                S0[j + 3] = fmaf(kq.w, ci, S0[j + 3]);
                y0[0] = fmaf(S0[j], qq.x, y0[0]);
                y0[1] = fmaf(S0[j + 1], qq.y, y0[1]);
                y0[2] = fmaf(S0[j + 2], qq.z, y0[2]);
                y0[3] = fmaf(S0[j + 3], qq.w, y0[3]);
            }
            G = Gn;
            const float o0 = halves((y0[0] + y0[1]) + (y0[2] + y0[3])) * G;
            // key half 0 writes the row: 32 consecutive outputs per wave
            if (hf == 0) IO<TI>::st(out, (tok * H + h) * N + i0, o0 * scale);
        }
        if (blk + 1 < nblk) store_block(buf ^ 1);
        __syncthreads();
    }
    if (s_out) {
#pragma unroll
        for (int j = 0; j < KH; j += 4)
            *(f32x4 *)(s_out + srow0 + j) = f32x4{S0[j] * G, S0[j + 1] * G, S0[j + 2] * G, S0[j + 3] * G};
    }
}

template <typename TI, int N>
hipError_t launch_typed_n(const GdnFwdArgs &a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.B * a.T * a.Hk;
    hipLaunchKernelGGL((gdn_norm_kernel<TI, N>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                       (const TI *)a.q, (const TI *)a.k, a.qn, a.kn, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // bf16 I/O: the chunk form on split-bf16 MFMA; other types token by token
    if constexpr (std::is_same<TI, uint16_t>::value) return launch_gdn_forward_cf(a, stream);
    hipLaunchKernelGGL((gdn_fwd_kernel<TI, N>), dim3((unsigned)((int64_t)a.B * a.H)), dim3(2 * N), 0, stream,
                       a.T, a.H, a.Hk, (const float *)a.qn, (const float *)a.kn, (const TI *)a.v, a.g, a.beta,
                       a.s0, (TI *)a.out, a.s_out);
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_typed(const GdnFwdArgs &a, hipStream_t stream) {
    return a.N == 128 ? launch_typed_n<TI, 128>(a, stream) : launch_typed_n<TI, 64>(a, stream);
}

}  // namespace

namespace {
template <typename TI>
hipError_t normalize_t(int N, const void *q, const void *k, float *qn, float *kn, int64_t rows, hipStream_t stream) {
    if (N == 128)
        hipLaunchKernelGGL((gdn_norm_kernel<TI, 128>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                           (const TI *)q, (const TI *)k, qn, kn, rows);
    else
        hipLaunchKernelGGL((gdn_norm_kernel<TI, 64>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                           (const TI *)q, (const TI *)k, qn, kn, rows);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gdn_normalize(int dtype, int N, const void *q, const void *k, float *qn, float *kn,
                                int64_t rows, hipStream_t stream) {
    if (dtype == 1) return normalize_t<uint16_t>(N, q, k, qn, kn, rows, stream);
    if (dtype == 2) return normalize_t<_Float16>(N, q, k, qn, kn, rows, stream);
    return normalize_t<float>(N, q, k, qn, kn, rows, stream);
}

hipError_t launch_gdn_forward(const GdnFwdArgs &a, hipStream_t stream) {
    if (a.dtype == 1) return launch_typed<uint16_t>(a, stream);
    if (a.dtype == 2) return launch_typed<_Float16>(a, stream);
    return launch_typed<float>(a, stream);
}

}  // namespace wkv7
