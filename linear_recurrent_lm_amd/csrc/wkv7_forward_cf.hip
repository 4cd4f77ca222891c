// WKV-7 forward in chunk form (C = 16) on FP32 MFMA, one lean workgroup per
// (sequence, head): N / 16 waves, wave w holding value rows 16 w .. 16 w + 15
// of the state in MFMA accumulators. Dense batches only.
//
// For a chunk with entering state S_0, gamma_t = prod_{u<=t} w_u (per key),
// sigma_s = prod_{u>s} w_u and x_t = S_{t-1} a_t, the recurrence
//     S_t = S_{t-1} diag(w_t) + x_t b_t^T + v_t k_t^T,   y_t = S_t r_t
// unrolls to
//     X = (I - L_ab)^-1 (A^ S_0^T + L_ak V)
//     Y = R^ S_0^T + M_rb X + M_rk V
//     S_16 = S_0 diag(gamma_15) + X^T B^ + V^T K^
// with A^_t = a_t gamma_{t-1}, R^_t = r_t gamma_t, B^_s = b_s sigma_s,
// K^_s = k_s sigma_s (products, never quotients), L_ab[t][s] = <a_t, b_s
// prod_{s<u<t} w_u> and L_ak the same with k (s < t), M_rb[t][s] = <r_t, b_s
// prod_{s<u<=t} w_u> and M_rk the same with k (s <= t).
//
// The four 16 x 16 matrices: when every decay of the chunk is at least 2^-6,
// gamma_15 >= 2^-96 and L_ab = A- B^^T, L_ak = A- K^^T, M_rb = R- B^^T,
// M_rk = R- K^^T with A- = A^ / gamma_15 and R- = R^ / gamma_15 exactly (each
// factor to rounding): four MFMA products. Other chunks form the entries as
// dot products with the decay products taken pair by pair (VALU). W =
// (I - L_ab)^-1 comes from forward substitution by one wave.
//
// Per chunk: stage r, w, k, a, b, v in LDS (fp32, w exponentiated for a
// log-decay input, tokens past the end as identity tokens) from registers
// loaded during the previous chunk; the prefix and suffix products and the
// scaled rows (one thread per key and row kind); the matrices and the dense
// products A^ S_0^T, R^ S_0^T; W and the right-hand sides; X, Y and the state
// update. Five LDS barriers per chunk. The workgroup uses 111 KB of LDS at
// N = 128 (one per CU, eight waves) and 60 KB at N = 64 (two per CU); the
// library uses it for dense batches at head size 128, where it replaces a
// token-order loop that runs the same flops on the VALU.
//
// MFMA layout (v_mfma_f32_16x16x4_f32): lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; element r of the result is D[4 (l / 16) + r][l % 16].
// The state tile T of a wave holds, in element r of lane l, S[16 w + l % 16]
// [16 T + 4 (l / 16) + r]: the output layout of the update product and the
// B-operand layout of A^ S_0^T when the contraction step (T, r) takes key
// 16 T + 4 g + r from lane group g = l / 16. Products over the 16 tokens take
// token 4 g + s at step s, which is element s of the D layout of X, rhs and Y.
#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr float kCfFastMinW = 0x1p-6f;

template <int N> struct CfLay {
    static constexpr int LD = N + 4;                     // row pitch of [16][N] rows
    static constexpr int TLD = 20;                       // row pitch of [N][16] key-major rows
    static constexpr int MLD = 17;                       // row pitch of 16 x 16 matrices
    static constexpr int IN = 0;                         // [6][16][LD] r w k a b v
    static constexpr int AH = IN + 6 * 16 * LD;          // [16][LD] A^
    static constexpr int RH = AH + 16 * LD;              // [16][LD] R^
    static constexpr int BH = RH + 16 * LD;              // [16][LD] B^
    static constexpr int KH = BH + 16 * LD;              // [16][LD] K^
    static constexpr int BT = KH + 16 * LD;              // [N][TLD] B^ by key
    static constexpr int KT = BT + N * TLD;              // [N][TLD] K^ by key
    static constexpr int MAT = KT + N * TLD;             // [5][16][MLD] L_ab L_ak M_rb M_rk W
    static constexpr int GAM = MAT + 5 * 16 * MLD;       // [N] gamma_15
    static constexpr int IGAM = GAM + N;                 // [N] 1 / gamma_15 (fast chunks)
    static constexpr int FLAG = IGAM + N;                // [N / 16] per-wave votes
    static constexpr int TOTAL = FLAG + N / 16;
};
enum { RR = 0, RW, RK, RA, RB, RV };
enum { MLAB = 0, MLAK, MMRB, MMRK, MW };

template <typename TI> struct Ld16;
template <> struct Ld16<uint16_t> { uint4 q; };
template <> struct Ld16<_Float16> { uint4 q; };
template <> struct Ld16<float> { float4 q; };
__device__ __forceinline__ void unpack16(const Ld16<uint16_t> &r, float *x) {
    const uint32_t u[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(u[e] << 16);
        x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack16(const Ld16<_Float16> &r, float *x) {
    const uint32_t u[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = half_lo(u[e]);
        x[2 * e + 1] = half_hi(u[e]);
    }
}
__device__ __forceinline__ void unpack16(const Ld16<float> &r, float *x) {
    x[0] = r.q.x; x[1] = r.q.y; x[2] = r.q.z; x[3] = r.q.w;
}

template <typename TI, int N>
__global__ __launch_bounds__(4 * N) void fwd_cf_kernel(FwdArgs p, int32_t units) {
    using L = CfLay<N>;
    constexpr int NT = 4 * N, NW = N / 16, NTILE = N / 16;
    constexpr int EPL = 16 / (int)sizeof(TI);            // elements per 16-byte load
    constexpr int GPR = N / EPL;                         // loads per row
    constexpr int LOADS = 6 * 16 * GPR / NT;             // loads per thread and chunk
    static_assert(6 * 16 * GPR % NT == 0, "whole loads per thread");
    extern __shared__ __align__(16) float sm[];

    const int unit = blockIdx.x;
    if (unit >= units) return;
    const int H = p.seg.H;
    const int h = unit % H, sq = unit / H;
    const Unit u = resolve_unit(p.seg, sq);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int row = 16 * wave + l16;                     // the lane's value row
    const int64_t ts = (int64_t)H * N;
    const int64_t base = (u.start * H + h) * N;
    const int64_t sbase = ((int64_t)sq * H + h) * (int64_t)(N * N);
    const int nch = (u.len + kChunk - 1) / kChunk;

    // the state: tile T, element r = S[row][16 T + 4 g + r]
    f32x4 S[NTILE];
#pragma unroll
    for (int T = 0; T < NTILE; ++T) {
        S[T] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.s0) {
            const float4 x = *(const float4 *)(p.s0 + sbase + (int64_t)row * N + 16 * T + 4 * g);
            S[T] = f32x4{x.x, x.y, x.z, x.w};
        }
    }

    const TI *srcs[6] = {(const TI *)p.r, (const TI *)p.w, (const TI *)p.k, (const TI *)p.a, (const TI *)p.b,
                         (const TI *)p.v};
    Ld16<TI> raw[LOADS];
    auto issue = [&](int c) {
        const int Lc = min(kChunk, u.len - c * kChunk);
        const int64_t t0 = (int64_t)c * kChunk;
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int i = q * NT + tid;
            const int s = i / (16 * GPR), e = (i / GPR) % 16, gq = i % GPR;
            raw[q] = *(const Ld16<TI> *)(srcs[s] + base + (t0 + min(e, Lc - 1)) * ts + gq * EPL);
        }
    };
    auto stage = [&](int c) {
        const int Lc = min(kChunk, u.len - c * kChunk);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int i = q * NT + tid;
            const int s = i / (16 * GPR), e = (i / GPR) % 16, gq = i % GPR;
            float x[EPL];
            unpack16(raw[q], x);
            if (s == RW) decay_of<EPL>(x, p.logw);
            if (e >= Lc) {                               // identity token past the end
#pragma unroll
                for (int k = 0; k < EPL; ++k) x[k] = s == RW ? 1.f : 0.f;
            }
            float *d = sm + L::IN + (s * 16 + e) * L::LD + gq * EPL;
#pragma unroll
            for (int k = 0; k < EPL; k += 4) *(float4 *)(d + k) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
        }
    };
    auto in_at = [&](int s, int t, int j) { return sm[L::IN + (s * 16 + t) * L::LD + j]; };

    if (nch > 0) issue(0);
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        const int Lc = min(kChunk, u.len - c * kChunk);
        const int64_t t0 = (int64_t)c * kChunk;
        lds_barrier();                                   // the previous chunk is done with LDS
        // ---- stage the chunk; the state entering it is its checkpoint
        stage(c);
        if (c + 1 < nch) issue(c + 1);
        if (p.ckpt) {
            float *ck = p.ckpt + ((u.ckpt + c) * H + h) * (int64_t)(N * N) + (int64_t)row * N + 4 * g;
#pragma unroll
            for (int T = 0; T < NTILE; ++T) *(float4 *)(ck + 16 * T) = make_float4(S[T][0], S[T][1], S[T][2], S[T][3]);
        }
        lds_barrier();
        // ---- prefix and suffix decay products of key j; part 0: A^, gamma_15
        //      and the fast-chunk vote, 1: R^, 2: B^, 3: K^
        {
            const int j = tid % N, part = tid / N;
            float wv[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) wv[t] = in_at(RW, t, j);
            bool ok = true;
            if (part == 0) {
                float gm = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    sm[L::AH + t * L::LD + j] = in_at(RA, t, j) * gm;
                    gm *= wv[t];
                    ok = ok && wv[t] >= kCfFastMinW;
                }
                sm[L::GAM + j] = gm;
                sm[L::IGAM + j] = 1.f / gm;
            } else if (part == 1) {
                float gm = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    gm *= wv[t];
                    sm[L::RH + t * L::LD + j] = in_at(RR, t, j) * gm;
                }
            } else {
                const int src = part == 2 ? RB : RK;
                float *rowm = sm + (part == 2 ? L::BH : L::KH);
                float *keym = sm + (part == 2 ? L::BT : L::KT) + j * L::TLD;
                float xs[16];
                float sg = 1.f;
#pragma unroll
                for (int s = 15; s >= 0; --s) {
                    xs[s] = in_at(src, s, j) * sg;
                    rowm[s * L::LD + j] = xs[s];
                    sg *= wv[s];
                }
                // by key: 16-byte stores (a pitch of 20 words puts 8 lanes'
                // stores on 32 distinct banks; single words would collide 8-way)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *(float4 *)(keym + 4 * q) = make_float4(xs[4 * q], xs[4 * q + 1], xs[4 * q + 2], xs[4 * q + 3]);
            }
            // one vote per wave (part 0 lanes decide; others agree)
            const bool all_ok = __all(ok);
            if (lane == 0) ((int *)sm)[L::FLAG + wave] = all_ok ? 1 : 0;
        }
        lds_barrier();
        bool fast = true;
#pragma unroll
        for (int q = 0; q < NW; ++q) fast = fast && ((const int *)sm)[L::FLAG + q] != 0;

        // ---- A^ S_0^T and R^ S_0^T for the wave's rows (D layout: element r
        //      = [token 4 g + r][row]); the four matrices
        f32x4 da = {0.f, 0.f, 0.f, 0.f}, dr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int T = 0; T < NTILE; ++T) {
            const float4 a4 = *(const float4 *)(sm + L::AH + l16 * L::LD + 16 * T + 4 * g);
            const float4 r4 = *(const float4 *)(sm + L::RH + l16 * L::LD + 16 * T + 4 * g);
            da = mfma4(a4.x, S[T][0], da); dr = mfma4(r4.x, S[T][0], dr);
            da = mfma4(a4.y, S[T][1], da); dr = mfma4(r4.y, S[T][1], dr);
            da = mfma4(a4.z, S[T][2], da); dr = mfma4(r4.z, S[T][2], dr);
            da = mfma4(a4.w, S[T][3], da); dr = mfma4(r4.w, S[T][3], dr);
        }
        if (fast) {
            // product pm (wave pm % NW): rows A- (pm < 2) or R-, columns B^ (even) or K^
            for (int pm = wave; pm < 4; pm += NW) {
                const float *lrow = sm + (pm < 2 ? L::AH : L::RH) + l16 * L::LD;
                const float *crow = sm + ((pm & 1) ? L::KH : L::BH) + l16 * L::LD;
                f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int T = 0; T < NTILE; ++T) {
                    const int j0 = 16 * T + 4 * g;
                    const float4 x4 = *(const float4 *)(lrow + j0), y4 = *(const float4 *)(crow + j0);
                    const float4 ig = *(const float4 *)(sm + L::IGAM + j0);
                    m = mfma4(x4.x * ig.x, y4.x, m);
                    m = mfma4(x4.y * ig.y, y4.y, m);
                    m = mfma4(x4.z * ig.z, y4.z, m);
                    m = mfma4(x4.w * ig.w, y4.w, m);
                }
                float *dst = sm + L::MAT + pm * 16 * L::MLD;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * g + r, s = l16;
                    const bool keep = pm < 2 ? s < t : s <= t;
                    dst[t * L::MLD + s] = keep ? m[r] : 0.f;
                }
            }
        } else {
            // entry by entry: slots (pm, t, s), the decay product pair by pair
            for (int e = tid; e < 4 * 256; e += NT) {
                const int pm = e >> 8, t = (e >> 4) & 15, s = e & 15;
                const bool isL = pm < 2;
                float acc = 0.f;
                if (isL ? s < t : s <= t) {
                    const int lr = isL ? RA : RR, cr = (pm & 1) ? RK : RB;
                    const int hi = isL ? t - 1 : t;      // decays of tokens s+1 .. hi
                    for (int j = 0; j < N; ++j) {
                        float d = 1.f;
                        for (int uu = s + 1; uu <= hi; ++uu) d *= in_at(RW, uu, j);
                        acc = fmaf(in_at(lr, t, j) * in_at(cr, s, j), d, acc);
                    }
                }
                sm[L::MAT + pm * 16 * L::MLD + t * L::MLD + s] = acc;
            }
        }
        lds_barrier();

        // ---- W = (I - L_ab)^-1 by forward substitution on wave 0: the quad
        //      of lanes 4 c .. 4 c + 3 owns column c, lane q of it the terms
        //      s = q mod 4 of W[t][c] = [t == c] + sum_{s<t} L_ab[t][s] W[s][c],
        //      completed by a quad sum; every wave: rhs = A^ S_0^T + L_ak V,
        //      Y = R^ S_0^T + M_rk V
        if (wave == 0) {
            const float *lab = sm + L::MAT + MLAB * 16 * L::MLD;
            const int cc = lane >> 2, qq = lane & 3;
            // L_ab[t][4 m + qq] for 4 m < t, read before the chain starts;
            // entries with s >= t are stored as zero and W entries not yet
            // formed are zero, so every term is taken without a test
            float lr[16][4];
#pragma unroll
            for (int t = 1; t < 16; ++t)
#pragma unroll
                for (int m = 0; 4 * m < t; ++m) lr[t][m] = lab[t * L::MLD + 4 * m + qq];
            float wq[4] = {0.f, 0.f, 0.f, 0.f};           // W[4 m + qq][cc]
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float x = (t == cc && qq == 0) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; 4 * m < t; ++m) x = fmaf(lr[t][m], wq[m], x);
                x = quad_sum(x);
                if ((t & 3) == qq) wq[t >> 2] = x;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) sm[L::MAT + MW * 16 * L::MLD + (4 * m + qq) * L::MLD + cc] = wq[m];
        }
        float vf[4];                                     // V[token 4 g + s][row]
#pragma unroll
        for (int s = 0; s < 4; ++s) vf[s] = in_at(RV, 4 * g + s, row);
        {
            const float *lak = sm + L::MAT + MLAK * 16 * L::MLD + l16 * L::MLD + 4 * g;
            const float *mrk = sm + L::MAT + MMRK * 16 * L::MLD + l16 * L::MLD + 4 * g;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                da = mfma4(lak[s], vf[s], da);
                dr = mfma4(mrk[s], vf[s], dr);
            }
        }
        lds_barrier();

        // ---- X = W rhs; Y += M_rb X; y out; S <- S diag(gamma_15) + X^T B^ + V^T K^
        f32x4 xx = {0.f, 0.f, 0.f, 0.f};
        {
            const float *wm = sm + L::MAT + MW * 16 * L::MLD + l16 * L::MLD + 4 * g;
#pragma unroll
            for (int s = 0; s < 4; ++s) xx = mfma4(wm[s], da[s], xx);
            const float *mrb = sm + L::MAT + MMRB * 16 * L::MLD + l16 * L::MLD + 4 * g;
#pragma unroll
            for (int s = 0; s < 4; ++s) dr = mfma4(mrb[s], xx[s], dr);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            if (t < Lc) IO<TI>::st((TI *)p.y, base + (t0 + t) * ts + row, dr[r]);
        }
#pragma unroll
        for (int T = 0; T < NTILE; ++T) {
            const float4 gm = *(const float4 *)(sm + L::GAM + 16 * T + 4 * g);
            f32x4 acc = f32x4{S[T][0] * gm.x, S[T][1] * gm.y, S[T][2] * gm.z, S[T][3] * gm.w};
            const float4 b4 = *(const float4 *)(sm + L::BT + (16 * T + l16) * L::TLD + 4 * g);
            const float4 k4 = *(const float4 *)(sm + L::KT + (16 * T + l16) * L::TLD + 4 * g);
            acc = mfma4(b4.x, xx[0], acc); acc = mfma4(k4.x, vf[0], acc);
            acc = mfma4(b4.y, xx[1], acc); acc = mfma4(k4.y, vf[1], acc);
            acc = mfma4(b4.z, xx[2], acc); acc = mfma4(k4.z, vf[2], acc);
            acc = mfma4(b4.w, xx[3], acc); acc = mfma4(k4.w, vf[3], acc);
            S[T] = acc;
        }
    }
    if (p.s_out) {
#pragma unroll
        for (int T = 0; T < NTILE; ++T)
            *(float4 *)(p.s_out + sbase + (int64_t)row * N + 16 * T + 4 * g) = make_float4(S[T][0], S[T][1], S[T][2], S[T][3]);
    }
}

template <typename TI, int N>
hipError_t launch_cf(const FwdArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)a.seg.B * a.seg.H;
    const size_t lds = (size_t)CfLay<N>::TOTAL * sizeof(float);
    hipError_t e = hipFuncSetAttribute((const void *)fwd_cf_kernel<TI, N>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fwd_cf_kernel<TI, N>), dim3((unsigned)units), dim3(4 * N), lds, stream, a, (int32_t)units);
    return hipGetLastError();
}

template <int N>
hipError_t launch_cf_n(const FwdArgs &a, hipStream_t stream) {
    if (a.dtype == 1) return launch_cf<uint16_t, N>(a, stream);
    if (a.dtype == 2) return launch_cf<_Float16, N>(a, stream);
    return launch_cf<float, N>(a, stream);
}

}  // namespace

hipError_t launch_forward_cf(const FwdArgs &a, int n, hipStream_t stream) {
    return n == 128 ? launch_cf_n<128>(a, stream) : launch_cf_n<64>(a, stream);
}

}  // namespace wkv7
