// WKV-7 forward, chunk-parallel form with FP32 MFMA for the dense products.
//
// The recurrence (RWKV-7 WKV-7; the model card's "chunked" path computes the
// same thing in a different operation order):
//     S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T + v_t k_t^T,   y_t = S_t r_t
// is advanced 16 tokens at a time. Within a chunk with entering state S_0,
// decays gamma_t = prod_{u<=t} w_u and D_{t,s} = prod_{s<u<=t} w_u, and
// x_t = S_{t-1} a_t, unrolling the recurrence gives
//     (I - L_ab) X = A^ S_0^T + L_ak V                (unit lower triangular)
//     Y            = R^ S_0^T + M_rb X + M_rk V
//     S_16         = S_0 diag(gamma_16) + X^T B^ + V^T K^
// with rows A^_t = gamma_{t-1} a_t, R^_t = gamma_t r_t, B^_s = D_{16,s} b_s,
// K^_s = D_{16,s} k_s and the 16x16 matrices
//     L_ab[t,s] = <a_t, b_s D_{t-1,s}>  (s < t)     M_rb[t,s] = <r_t, b_s D_{t,s}>  (s <= t)
// (L_ak, M_rk the same with k_s). The two dense contractions [A^;R^] S_0^T
// (32x64x64) and [X|V]^T [B^;K^] (64x64x32) run on v_mfma_f32_16x16x4_f32;
// everything else is VALU.
//
// The 16x16 matrices are built as dot products of precomputed rows using
// 4-token sub-chunks: for t in sub-chunk p and s in an earlier sub-chunk q the
// decay factorises division-free as D_{t-1,s} = [prod_{4p<=u<t} w_u] *
// [prod_{s<u<4p} w_u]; for s in the same sub-chunk the within-sub-chunk
// prefix F_s = prod_{4p<=u<=s} w_u is divided out, with every factor of F
// clamped to >= 2^-30 so F >= 2^-120 stays a normal fp32 number (w = 0
// then acts as 2^-30 on at most three neighbouring tokens of one sub-chunk).
// The chunk-level decays (gamma, D_{16,s}) are exact products.
//
// Layout and work split: one 256-thread workgroup (4 waves) per (sequence,
// head, block of RB value rows); value rows are independent, so a unit may be
// split in 1, 2 or 4 row blocks to fill the machine. The state block lives in
// the MFMA accumulators as S^T tiles: lane l of a wave holds
// S[i0 + 16*it + l%16][16*jt + 4*(l/16) + r], r = 0..3, which is directly the
// B operand of the next chunk's [A^;R^] S_0^T product. Inputs are staged to
// LDS as fp32 with one 16-byte load per 8 bf16 values.
#include "wkv7_kernels.h"

namespace wkv7 {
namespace {

constexpr int kThreads = 256;
constexpr int QLD = 68;    // row stride (floats) of Q and the C x C operand rows
constexpr int KLD = 36;    // row stride of the transposed [B^;K^] and [X|V] tiles
constexpr float kMinFactor = 9.313225746154785e-10f;  // 2^-30

// LDS layout (floats).
template <int RB>
struct Lay {
    static constexpr int IN = 0;                       // [5][16][64]: r w k a b
    static constexpr int P = 0;                        // alias [WPI][32][RB]
    static constexpr int LM = 2048;                    // alias [4][16][16]
    static constexpr int Q = 5 * 16 * 64;              // [32][QLD]: A^, R^
    static constexpr int BKT = Q + 32 * QLD;           // [64][KLD]: B^ | K^ (by column j)
    static constexpr int XVT = BKT + 64 * KLD;         // [RB][KLD]: X | V (by row i)
    static constexpr int AR = XVT + RB * KLD;          // [32][QLD]: A' (a), A' (r)
    static constexpr int BV = AR + 32 * QLD;           // [40][QLD]: b versions
    static constexpr int KV = BV + 40 * QLD;           // [40][QLD]: k versions
    static constexpr int GC = KV + 40 * QLD;           // [64]: gamma_16
    static constexpr int TOTAL = GC + 64;
};

enum { IR = 0, IW, IK, IA, IB };

__device__ __forceinline__ int ver_off(int p) { return 2 * p * (p + 1); }

// Raw chunk data in flight: 3 vectors of 8 elements per thread.
template <typename TI> struct Raw;
template <> struct Raw<uint16_t> { uint4 q[3]; };
template <> struct Raw<float> { float4 q[3][2]; };

__device__ __forceinline__ void raw_load(const uint16_t *p, Raw<uint16_t> &r, int k) {
    r.q[k] = *(const uint4 *)p;
}
__device__ __forceinline__ void raw_load(const float *p, Raw<float> &r, int k) {
    r.q[k][0] = *(const float4 *)p;
    r.q[k][1] = *(const float4 *)(p + 4);
}
__device__ __forceinline__ void raw_unpack(const Raw<uint16_t> &r, int k, float *x) {
    const uint32_t u[4] = {r.q[k].x, r.q[k].y, r.q[k].z, r.q[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(u[e] << 16);
        x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void raw_unpack(const Raw<float> &r, int k, float *x) {
    x[0] = r.q[k][0].x; x[1] = r.q[k][0].y; x[2] = r.q[k][0].z; x[3] = r.q[k][0].w;
    x[4] = r.q[k][1].x; x[5] = r.q[k][1].y; x[6] = r.q[k][1].z; x[7] = r.q[k][1].w;
}

// Rows b_s * V^(p)_s and k_s * V^(p)_s of source sub-chunk Q for every target
// sub-chunk p >= Q: for p > Q the division-free decay prod_{s<u<4p} w_u, for
// p = Q the reciprocal of the clamped within-sub-chunk prefix F_s.
template <int Q>
__device__ __forceinline__ void b_k_versions(const float *wv, const float *W, const float *s_in,
                                             float *s_BV, float *s_KV, int j) {
    float suf[4];
    suf[3] = 1.f;
    suf[2] = wv[4 * Q + 3];
    suf[1] = wv[4 * Q + 2] * suf[2];
    suf[0] = wv[4 * Q + 1] * suf[1];
    float F = 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int s = 4 * Q + e;
        F *= fmaxf(wv[s], 9.313225746154785e-10f);
        const float bs = s_in[4 * 1024 + s * 64 + j];
        const float ks = s_in[2 * 1024 + s * 64 + j];
        const float inv = __builtin_amdgcn_rcpf(F);
        s_BV[(2 * Q * (Q + 1) + s) * 68 + j] = bs * inv;
        s_KV[(2 * Q * (Q + 1) + s) * 68 + j] = ks * inv;
        float m = suf[e];
#pragma unroll
        for (int pp = Q + 1; pp < 4; ++pp) {
            s_BV[(2 * pp * (pp + 1) + s) * 68 + j] = bs * m;
            s_KV[(2 * pp * (pp + 1) + s) * 68 + j] = ks * m;
            m *= W[pp];
        }
    }
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TI, int NIT>
__global__ __launch_bounds__(kThreads, 2) void fwd_chunk_kernel(FwdArgs p, int32_t units) {
    constexpr int RB = 16 * NIT;       // value rows per workgroup
    constexpr int NRB = 4 / NIT;       // row blocks per unit
    constexpr int WPI = 4 / NIT;       // waves sharing one 16-row tile (K split of D1)
    constexpr int JPW = NIT;           // 16-column tiles of the state per wave
    using LY = Lay<RB>;
    extern __shared__ __align__(16) float sm[];

    // Workgroup -> (unit, row block). Row blocks of one unit go to the same
    // XCD (workgroups are dealt to the 8 XCDs round robin) so that their
    // shared reads of r, w, k, a, b hit one L2.
    int unit, rb;
    if (NRB == 1) {
        unit = blockIdx.x;
        rb = 0;
    } else {
        const int g = blockIdx.x / (8 * NRB), wq = blockIdx.x % (8 * NRB);
        unit = g * 8 + (wq & 7);
        rb = wq >> 3;
    }
    if (unit >= units) return;
    const int H = p.seg.H;
    const int h = unit % H;
    const int sq = unit / H;
    const Unit u = resolve_unit(p.seg, sq);
    const int i0 = rb * RB;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kq = lane >> 4;
    const int it = wave % NIT, jg = wave / NIT;
    const int irow = 16 * it + l16;                      // local value row of this lane

    const int64_t ts = (int64_t)H * kN;
    const int64_t base = (u.start * H + h) * kN;
    const int64_t sbase = ((int64_t)sq * H + h) * (kN * kN);

    // State tiles: acc[q][r] = S[i0 + irow][16*jt + 4*kq + r], jt = jg*JPW + q.
    f32x4 acc[JPW];
#pragma unroll
    for (int q = 0; q < JPW; ++q) {
        const int jt = jg * JPW + q;
        if (p.s0) {
            const float4 v4 = *(const float4 *)(p.s0 + sbase + (int64_t)(i0 + irow) * kN + 16 * jt + 4 * kq);
            acc[q] = f32x4{v4.x, v4.y, v4.z, v4.w};
        } else {
            acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    float *s_in = sm + LY::IN;
    float *s_P = sm + LY::P;
    float *s_L = sm + LY::LM;
    float *s_Q = sm + LY::Q;
    float *s_BKt = sm + LY::BKT;
    float *s_XVt = sm + LY::XVT;
    float *s_AR = sm + LY::AR;
    float *s_BV = sm + LY::BV;
    float *s_KV = sm + LY::KV;
    float *s_gC = sm + LY::GC;

    const int nch = (u.len + kChunk - 1) / kChunk;
    Raw<TI> raw;
    // Thread tid stages element group q = tid + 256k: stream 2k + (tid >> 7)
    // (uniform per wave), token (q >> 3) & 15, elements 8*(q & 7) .. +7.
    const int half = __builtin_amdgcn_readfirstlane(tid >> 7);
    const TI *sp0 = (const TI *)(half ? p.w : p.r);
    const TI *sp1 = (const TI *)(half ? p.a : p.k);
    const TI *sp2 = (const TI *)(half ? p.v : p.b);
    auto issue = [&](int cc) {
        const int Lc = min(kChunk, u.len - cc * kChunk);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int q = tid + k * kThreads;
            const int t = (q >> 3) & 15, e0 = (q & 7) * 8;
            const TI *sp = k == 0 ? sp0 : k == 1 ? sp1 : sp2;
            if (t < Lc) raw_load(sp + base + (int64_t)(cc * kChunk + t) * ts + e0, raw, k);
        }
    };
    if (nch > 0) issue(0);
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        const int t0 = c * kChunk;
        const int L = min(kChunk, u.len - t0);
        __syncthreads();

        // ---- stage chunk c from registers (identity tokens w=1, rest 0, past the end),
        //      then start the loads of chunk c+1
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int q = tid + k * kThreads;
            const int st = q >> 7, t = (q >> 3) & 15, e0 = (q & 7) * 8;
            float x[8];
            if (t < L) {
                raw_unpack(raw, k, x);
            } else {
                const float f = st == IW ? 1.f : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = f;
            }
            if (st < 5) {
                float *d = s_in + (st * 16 + t) * 64 + e0;
                *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
                *(float4 *)(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int row = e0 + e - i0;
                    if (row >= 0 && row < RB) s_XVt[row * KLD + 16 + t] = x[e];
                }
            }
        }
        if (c + 1 < nch) issue(c + 1);
        if (p.ckpt) {
            float *cp = p.ckpt + ((u.ckpt + c) * H + h) * (int64_t)(kN * kN) + (int64_t)(i0 + irow) * kN;
#pragma unroll
            for (int q = 0; q < JPW; ++q) {
                const int jt = jg * JPW + q;
                *(float4 *)(cp + 16 * jt + 4 * kq) = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
            }
        }
        __syncthreads();

        // ---- decays and operand rows (4 threads per key column j)
        {
            const int role = tid >> 6, j = tid & 63;
            const float *w_ = s_in + IW * 1024 + j;
            if (role == 0) {            // A^, R^ and gamma_16
                float g = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    s_Q[t * QLD + j] = s_in[IA * 1024 + t * 64 + j] * g;
                    g *= w_[t * 64];
                    s_Q[(16 + t) * QLD + j] = s_in[IR * 1024 + t * 64 + j] * g;
                }
                s_gC[j] = g;
            } else if (role == 1) {     // B^, K^ (transposed for the MFMA A operand)
                float d = 1.f;
#pragma unroll
                for (int s = 15; s >= 0; --s) {
                    s_BKt[j * KLD + s] = s_in[IB * 1024 + s * 64 + j] * d;
                    s_BKt[j * KLD + 16 + s] = s_in[IK * 1024 + s * 64 + j] * d;
                    d *= w_[s * 64];
                }
            } else {
                // roles 2 and 3: b, k versions per target sub-chunk (role 3: source
                // sub-chunks 0 and 1; role 2: 2 and 3, plus the prefix rows
                // A' = a F_{t-1}, R' = r F_t)
                float wv[16], W[4];
#pragma unroll
                for (int t = 0; t < 16; ++t) wv[t] = w_[t * 64];
#pragma unroll
                for (int sc = 0; sc < 4; ++sc)
                    W[sc] = (wv[4 * sc] * wv[4 * sc + 1]) * (wv[4 * sc + 2] * wv[4 * sc + 3]);
                if (role == 2) {
#pragma unroll
                    for (int sc = 0; sc < 4; ++sc) {
                        float f = 1.f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = 4 * sc + e;
                            s_AR[t * QLD + j] = s_in[IA * 1024 + t * 64 + j] * f;
                            f *= fmaxf(wv[t], kMinFactor);
                            s_AR[(16 + t) * QLD + j] = s_in[IR * 1024 + t * 64 + j] * f;
                        }
                    }
                }
                if (role == 3) {
                    b_k_versions<0>(wv, W, s_in, s_BV, s_KV, j);
                    b_k_versions<1>(wv, W, s_in, s_BV, s_KV, j);
                } else {
                    b_k_versions<2>(wv, W, s_in, s_BV, s_KV, j);
                    b_k_versions<3>(wv, W, s_in, s_BV, s_KV, j);
                }
            }
        }
        __syncthreads();

        // ---- D1 on MFMA: P[t'][i] = sum_j Q[t'][j] S_0[i][j] over this wave's
        //      column tiles (a K split when several waves share one row tile)
        f32x4 d1[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            d1[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < JPW; ++q) {
                const int jt = jg * JPW + q;
                const float4 a4 = *(const float4 *)(s_Q + (16 * tt + l16) * QLD + 16 * jt + 4 * kq);
                d1[tt] = mfma4(a4.x, acc[q][0], d1[tt]);
                d1[tt] = mfma4(a4.y, acc[q][1], d1[tt]);
                d1[tt] = mfma4(a4.z, acc[q][2], d1[tt]);
                d1[tt] = mfma4(a4.w, acc[q][3], d1[tt]);
            }
            if (WPI > 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s_P[(jg * 32 + 16 * tt + 4 * kq + r) * RB + irow] = d1[tt][r];
            }
        }

        // ---- 16x16 matrices on VALU: 120 L items and 136 M items, one per thread
        {
            int t, s, mat;
            if (tid < 120) {
                t = 1;
                while ((t + 1) * t / 2 <= tid) ++t;
                s = tid - t * (t - 1) / 2;
                mat = 0;
            } else {
                const int mi = tid - 120;
                t = 0;
                while ((t + 1) * (t + 2) / 2 <= mi) ++t;
                s = mi - t * (t + 1) / 2;
                mat = 1;
            }
            const int vrow = ver_off(t >> 2) + s;
            const float *ar = s_AR + (16 * mat + t) * QLD;
            const float *bv = s_BV + vrow * QLD;
            const float *kv = s_KV + vrow * QLD;
            float db0 = 0.f, db1 = 0.f, dk0 = 0.f, dk1 = 0.f;
#pragma unroll
            for (int j = 0; j < 64; j += 8) {
                const float4 x0 = *(const float4 *)(ar + j), x1 = *(const float4 *)(ar + j + 4);
                const float4 b0 = *(const float4 *)(bv + j), b1 = *(const float4 *)(bv + j + 4);
                const float4 k0 = *(const float4 *)(kv + j), k1 = *(const float4 *)(kv + j + 4);
                db0 = fmaf(x0.x, b0.x, db0); db1 = fmaf(x0.y, b0.y, db1);
                db0 = fmaf(x0.z, b0.z, db0); db1 = fmaf(x0.w, b0.w, db1);
                db0 = fmaf(x1.x, b1.x, db0); db1 = fmaf(x1.y, b1.y, db1);
                db0 = fmaf(x1.z, b1.z, db0); db1 = fmaf(x1.w, b1.w, db1);
                dk0 = fmaf(x0.x, k0.x, dk0); dk1 = fmaf(x0.y, k0.y, dk1);
                dk0 = fmaf(x0.z, k0.z, dk0); dk1 = fmaf(x0.w, k0.w, dk1);
                dk0 = fmaf(x1.x, k1.x, dk0); dk1 = fmaf(x1.y, k1.y, dk1);
                dk0 = fmaf(x1.z, k1.z, dk0); dk1 = fmaf(x1.w, k1.w, dk1);
            }
            // row-major 16x16: [0] L_ab, [1] L_ak, [2] M_rb, [3] M_rk (upper parts zero)
            s_L[(2 * mat) * 256 + t * 16 + s] = db0 + db1;
            s_L[(2 * mat + 1) * 256 + t * 16 + s] = dk0 + dk1;
        }
        __syncthreads();
        float *s_Lab = s_L, *s_Lak = s_L + 256, *s_Mrb = s_L + 512, *s_Mrk = s_L + 768;
        float *s_Wi = s_L + 1024;                 // (I - L_ab)^-1, row-major
        float *s_Y = s_L + 1280;                  // [16][RB] output tile

        // ---- (I - L_ab)^-1 by column-oriented substitution (16 threads); the
        //      strictly upper parts of the four matrices are cleared meanwhile
        if (tid < 16) {
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) x[t] = t == tid ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 15; ++s2) {
#pragma unroll
                for (int t = s2 + 1; t < 16; ++t) x[t] = fmaf(s_Lab[t * 16 + s2], x[s2], x[t]);
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) s_Wi[t * 16 + tid] = x[t];
        } else if (tid >= 64 && tid < 64 + 4 * 16) {
            const int m = (tid - 64) >> 4, row = tid & 15;
            const int first = (m == 0 || m == 1) ? row : row + 1;   // L: s >= t, M: s > t
            for (int c2 = first; c2 < 16; ++c2) s_L[m * 256 + row * 16 + c2] = 0.f;
        }
        if (WPI > 1) {
            for (int q = tid; q < 32 * RB; q += kThreads) {
                float acc0 = s_P[q];
#pragma unroll
                for (int g = 1; g < WPI; ++g) acc0 += s_P[g * 32 * RB + q];
                s_P[q] = acc0;
            }
        }
        __syncthreads();

        // ---- per 16-row tile (one owner wave): rhs = P_a + L_ak V; X = W rhs;
        //      Y = P_r + M_rk V + M_rb X, all on MFMA; the 16x16 output layout
        //      is the B-operand layout of the next product
        if (jg == 0) {
            f32x4 pa = d1[0], pr = d1[1];
            if (WPI > 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pa[r] = s_P[(4 * kq + r) * RB + irow];
                    pr[r] = s_P[(16 + 4 * kq + r) * RB + irow];
                }
            }
            const float4 v4 = *(const float4 *)(s_XVt + irow * KLD + 16 + 4 * kq);
            const float vb[4] = {v4.x, v4.y, v4.z, v4.w};
            const float4 lak = *(const float4 *)(s_Lak + l16 * 16 + 4 * kq);
            const float4 mrk = *(const float4 *)(s_Mrk + l16 * 16 + 4 * kq);
            const float4 wi = *(const float4 *)(s_Wi + l16 * 16 + 4 * kq);
            const float4 mrb = *(const float4 *)(s_Mrb + l16 * 16 + 4 * kq);
            pa = mfma4(lak.x, vb[0], pa); pa = mfma4(lak.y, vb[1], pa);
            pa = mfma4(lak.z, vb[2], pa); pa = mfma4(lak.w, vb[3], pa);
            pr = mfma4(mrk.x, vb[0], pr); pr = mfma4(mrk.y, vb[1], pr);
            pr = mfma4(mrk.z, vb[2], pr); pr = mfma4(mrk.w, vb[3], pr);
            f32x4 xx = {0.f, 0.f, 0.f, 0.f};
            xx = mfma4(wi.x, pa[0], xx); xx = mfma4(wi.y, pa[1], xx);
            xx = mfma4(wi.z, pa[2], xx); xx = mfma4(wi.w, pa[3], xx);
            pr = mfma4(mrb.x, xx[0], pr); pr = mfma4(mrb.y, xx[1], pr);
            pr = mfma4(mrb.z, xx[2], pr); pr = mfma4(mrb.w, xx[3], pr);
            *(float4 *)(s_XVt + irow * KLD + 4 * kq) = make_float4(xx[0], xx[1], xx[2], xx[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) s_Y[(4 * kq + r) * RB + irow] = pr[r];
        }
        __syncthreads();

        // ---- store y for the real tokens (consecutive threads, consecutive channels)
        for (int q = tid; q < L * RB; q += kThreads) {
            const int t = q / RB, il = q - t * RB;
            IO<TI>::st((TI *)p.y, base + (int64_t)(t0 + t) * ts + i0 + il, s_Y[q]);
        }

        // ---- D2 on MFMA: S^T[j][i] = gamma[j] S_0^T[j][i] + sum_k BK[k][j] XV[k][i]
        {
            const float *xr = s_XVt + irow * KLD + 4 * kq;
            const float4 xa = *(const float4 *)xr, va = *(const float4 *)(xr + 16);
#pragma unroll
            for (int q = 0; q < JPW; ++q) {
                const int jt = jg * JPW + q;
                const float4 g4 = *(const float4 *)(s_gC + 16 * jt + 4 * kq);
                acc[q][0] *= g4.x; acc[q][1] *= g4.y; acc[q][2] *= g4.z; acc[q][3] *= g4.w;
                const float *br = s_BKt + (16 * jt + l16) * KLD + 4 * kq;
                const float4 b0 = *(const float4 *)br, k0 = *(const float4 *)(br + 16);
                acc[q] = mfma4(b0.x, xa.x, acc[q]);
                acc[q] = mfma4(b0.y, xa.y, acc[q]);
                acc[q] = mfma4(b0.z, xa.z, acc[q]);
                acc[q] = mfma4(b0.w, xa.w, acc[q]);
                acc[q] = mfma4(k0.x, va.x, acc[q]);
                acc[q] = mfma4(k0.y, va.y, acc[q]);
                acc[q] = mfma4(k0.z, va.z, acc[q]);
                acc[q] = mfma4(k0.w, va.w, acc[q]);
            }
        }
    }

    if (p.s_out) {
        float *op = p.s_out + sbase + (int64_t)(i0 + irow) * kN;
#pragma unroll
        for (int q = 0; q < JPW; ++q) {
            const int jt = jg * JPW + q;
            *(float4 *)(op + 16 * jt + 4 * kq) = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
        }
    }
}

template <typename TI, int NIT>
hipError_t launch_chunk(const FwdArgs &a, int32_t units, hipStream_t stream) {
    constexpr int NRB = 4 / NIT;
    const size_t lds = (size_t)Lay<16 * NIT>::TOTAL * sizeof(float);
    auto fn = fwd_chunk_kernel<TI, NIT>;
    hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t blocks = NRB == 1 ? units : ((int64_t)units + 7) / 8 * 8 * NRB;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), lds, stream, a, units);
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_typed(const FwdArgs &a, hipStream_t stream) {
    const int S = a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B;
    const int32_t units = S * a.seg.H;
    // Split value rows across workgroups when there are too few units to
    // give every CU two workgroups.
    if (units >= 512) return launch_chunk<TI, 4>(a, units, stream);
    if (units >= 256) return launch_chunk<TI, 2>(a, units, stream);
    return launch_chunk<TI, 1>(a, units, stream);
}

}  // namespace

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream) {
    return a.dtype == 1 ? launch_typed<uint16_t>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace wkv7
