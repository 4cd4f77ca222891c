// WKV-7 backward, second pass: per-chunk gradients on FP32 MFMA.
//
// Forward recurrence (RWKV-7 WKV-7): S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T
// + v_t k_t^T, y_t = S_t r_t. Gradients of L = sum <dy, y> + <ds_out, S_T>.
// Each chunk starts from its stored checkpoint S_0 (the state entering the
// chunk) and from dS_C, the gradient of the state leaving it, written by the
// first pass (the state-gradient sweep); with both given, chunks are
// independent and run in parallel, kChunksPerGroup consecutive chunks per
// workgroup. Nothing is reconstructed by dividing by w.
//
// Within a chunk the forward is (tokens t = 0..15, as in the forward kernel)
//     X = W (A^ S_0^T + L_ak V),  W = (I - L_ab)^-1
//     Y = R^ S_0^T + M_rb X + M_rk V
//     S_C = S_0 diag(gamma_C) + X^T B^ + V^T K^
// and its reverse mode is
//     dX   = B^ dS_C^T + M_rb^T dY          drhs = W^T dX
//     dV   = K^ dS_C^T + M_rk^T dY + L_ak^T drhs
//     dA^ = drhs S_0, dR^ = dY S_0, dB^ = X dS_C, dK^ = V dS_C
//     dL_ab = drhs X^T, dL_ak = drhs V^T (strictly lower), dM_rb = dY X^T,
//     dM_rk = dY V^T (lower)
// followed by the chain rule through the decay products. The 16x16 matrices
// use the forward's 4-token sub-chunk factorisation (rows A' = a F_ex,
// R' = r F_in and b/k "versions" b_s V_s, k_s V_s), so their gradients with
// respect to r, a, b, k are weighted sums of those rows. The decay gradient
// is assembled as u_m = w_m dw_m from the log-derivatives of every product
// that contains w_m (prefix gamma, suffix D_{15,s}, and the pair decays of
// the 16x16 matrices, whose contribution is a sum over the (s, t) pairs that
// straddle m), then dw = u / w. The whole backward uses w' = max(w, 2^-30),
// so dw is finite at w = 0 and equals the gradient there to within the clamp.
//
// One 512-thread workgroup (8 waves) per (sequence, head, chunk group). 16x64
// chunk matrices and the two 64x64 states live in LDS, row-major; MFMA
// operands are 16-byte loads along the contraction index where the layout
// allows it. Waves w and w+4 share a SIMD and take complementary (MFMA and
// VALU) work in each phase.
#include "wkv7_kernels.h"

namespace wkv7 {
namespace {

constexpr int kThreads = 512;
constexpr int kChunksPerGroup = 8;                // chunks per workgroup (consecutive)
constexpr int LD = 68;                            // row pitch of 16x64 / 64x64 arrays
constexpr float kMinW = 9.313225746154785e-10f;   // 2^-30

// LDS layout (floats)
constexpr int O_IN = 0;                      // [7][16][LD] r w k a b v dy
constexpr int O_Q = O_IN + 7 * 16 * LD;         // [32][LD] A^ (0..15), R^ (16..31)
constexpr int O_BK = O_Q + 32 * LD;          // [32][LD] B^, K^
constexpr int O_AR = O_BK + 32 * LD;         // [32][LD] A', R'
constexpr int O_BV = O_AR + 32 * LD;         // [40][LD] b versions
constexpr int O_KV = O_BV + 40 * LD;         // [40][LD] k versions
constexpr int O_VV = O_KV + 40 * LD;         // [40][LD] bare decay versions
constexpr int O_S0 = O_VV + 40 * LD;         // [64][LD] S_0
constexpr int O_DS = O_S0 + 64 * LD;         // [64][LD] dS_C
constexpr int O_X = O_DS + 64 * LD;          // [16][LD] X[t][i]
constexpr int O_DR = O_X + 16 * LD;          // [16][LD] drhs[t][i]
constexpr int O_G = O_DR + 16 * LD;          // [4][16][LD] dA^, dR^, dB^, dK^ ([t][j])
constexpr int O_M = O_G + 64 * LD;           // [9][256] Lab Lak Mrb Mrk W dLab dLak dMrb dMrk
constexpr int O_GC = O_M + 9 * 256;          // [64] gamma_C
constexpr int O_DGC = O_GC + 64;             // [64] d gamma_C
constexpr int LDS_FLOATS = O_DGC + 64;
static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");

enum { IR = 0, IW, IK, IA, IB, IV, IDY };
enum { MLAB = 0, MLAK, MMRB, MMRK, MW, MDLAB, MDLAK, MDMRB, MDMRK };

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int ver_off(int p) { return 2 * p * (p + 1); }

// acc[m][n] += sum_k A[m][k] B[k][n] with A row-major (pitch lda) and B given
// transposed, Bt[n][k] row-major (pitch ldb): both operands 16-byte loads.
__device__ __forceinline__ f32x4 mm_AtBt(f32x4 acc, const float *A, int lda, const float *Bt, int ldb,
                                         int l16, int kq, int kdim) {
    for (int k0 = 0; k0 < kdim; k0 += 16) {
        const float4 a = *(const float4 *)(A + l16 * lda + k0 + 4 * kq);
        const float4 b = *(const float4 *)(Bt + l16 * ldb + k0 + 4 * kq);
        acc = mfma4(a.x, b.x, acc); acc = mfma4(a.y, b.y, acc);
        acc = mfma4(a.z, b.z, acc); acc = mfma4(a.w, b.w, acc);
    }
    return acc;
}

// acc += A B with A row-major (16-byte loads along k) and B row-major [k][n]
// (scalar loads; consecutive lanes read consecutive n).
__device__ __forceinline__ f32x4 mm_AtB(f32x4 acc, const float *A, int lda, const float *B, int ldb,
                                        int l16, int kq, int kdim) {
    for (int k0 = 0; k0 < kdim; k0 += 16) {
        const float4 a = *(const float4 *)(A + l16 * lda + k0 + 4 * kq);
        const float *bp = B + (k0 + 4 * kq) * ldb + l16;
        acc = mfma4(a.x, bp[0], acc); acc = mfma4(a.y, bp[ldb], acc);
        acc = mfma4(a.z, bp[2 * ldb], acc); acc = mfma4(a.w, bp[3 * ldb], acc);
    }
    return acc;
}

// acc += A^T B for A = [k][m], B = [k][n] row-major with 16 rows k.
__device__ __forceinline__ f32x4 mm_TB(f32x4 acc, const float *A, int lda, const float *B, int ldb,
                                       int l16, int kq) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int k = 4 * kq + e;
        acc = mfma4(A[k * lda + l16], B[k * ldb + l16], acc);
    }
    return acc;
}

template <typename TI> struct Raw;
template <> struct Raw<uint16_t> { uint4 q[2]; };
template <> struct Raw<float> { float4 q[2][2]; };

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

// Version rows of source sub-chunk Q (b_s V, k_s V and the bare factor V) for
// every target sub-chunk p >= Q; V = prod_{s<u<4p} w_u for p > Q, 1 / F_s for p = Q.
template <int Q>
__device__ __forceinline__ void versions(const float *wv, const float *W, const float *s_in,
                                         float *s_bv, float *s_kv, float *s_vv, int j) {
    float suf[4];
    suf[3] = 1.f;
    suf[2] = wv[4 * Q + 3];
    suf[1] = wv[4 * Q + 2] * suf[2];
    suf[0] = wv[4 * Q + 1] * suf[1];
    float F = 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int s = 4 * Q + e;
        F *= wv[s];
        const float bs = s_in[(IB * 16 + s) * LD + j];
        const float ks = s_in[(IK * 16 + s) * LD + j];
        const float inv = __builtin_amdgcn_rcpf(F);
        const int r0 = (ver_off(Q) + s) * LD + j;
        s_vv[r0] = inv;
        s_bv[r0] = bs * inv;
        s_kv[r0] = ks * inv;
        float m = suf[e];
#pragma unroll
        for (int pp = Q + 1; pp < 4; ++pp) {
            const int r1 = (ver_off(pp) + s) * LD + j;
            s_vv[r1] = m;
            s_bv[r1] = bs * m;
            s_kv[r1] = ks * m;
            m *= W[pp];
        }
    }
}

struct AsmArgs {
    const float *s_in, *s_AR, *s_BV, *s_KV, *s_VV, *s_G, *s_M, *s_dgC;
    float *s_U;          // [8][16][LD] partial pair parts of u (aliases S_0 and dS_C)
    int j, wave;
};

// Pair parts for rows t in {T0, T1} of key column j: the prefix sums over s
// of zl_s = dL_ab[t,s] b_s V + dL_ak[t,s] k_s V and zm_s (same with dM) give
// the da_t, dr_t pair parts and the straddling-pair part of u (A'_t zl_s for
// s < m < t, R'_t zm_s for s < m <= t); db_s, dk_s pair parts for s in {T0, T1}.
template <int T0, int T1>
__device__ __forceinline__ void assemble_rows(const AsmArgs &g, float (&st5)[2][5]) {
    constexpr int TK[2] = {T0, T1};
    const int j = g.j;
    const float *Mdlab = g.s_M + MDLAB * 256, *Mdlak = g.s_M + MDLAK * 256;
    const float *Mdmrb = g.s_M + MDMRB * 256, *Mdmrk = g.s_M + MDMRK * 256;
    float um[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) um[m] = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = TK[q];
        const int pv = ver_off(t >> 2);
        const float ap = g.s_AR[t * LD + j], rp = g.s_AR[(16 + t) * LD + j];
        float cl = 0.f, cm = 0.f;
#pragma unroll
        for (int s = 0; s <= t; ++s) {
            const float bvs = g.s_BV[(pv + s) * LD + j], kvs = g.s_KV[(pv + s) * LD + j];
            if (s < t) cl += Mdlab[t * 16 + s] * bvs + Mdlak[t * 16 + s] * kvs;
            cm += Mdmrb[t * 16 + s] * bvs + Mdmrk[t * 16 + s] * kvs;
            if (s + 1 < t) um[s + 1] = fmaf(ap, cl, um[s + 1]);
            if (s + 1 <= t && s + 1 < 16) um[s + 1] = fmaf(rp, cm, um[s + 1]);
        }
        st5[q][2] = cl;          // da pair part (times F_ex later)
        st5[q][0] = cm;          // dr pair part (times F_in later)
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) g.s_U[(g.wave * 16 + m) * LD + j] = um[m];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int s = TK[q];
        float accb = 0.f, acck = 0.f;
#pragma unroll
        for (int t = s; t < 16; ++t) {
            const float vv = g.s_VV[(ver_off(t >> 2) + s) * LD + j];
            const float ap = g.s_AR[t * LD + j], rp = g.s_AR[(16 + t) * LD + j];
            const float cb = (t > s ? Mdlab[t * 16 + s] * ap : 0.f) + Mdmrb[t * 16 + s] * rp;
            const float ck = (t > s ? Mdlak[t * 16 + s] * ap : 0.f) + Mdmrk[t * 16 + s] * rp;
            accb = fmaf(cb, vv, accb);
            acck = fmaf(ck, vv, acck);
        }
        st5[q][3] = accb;
        st5[q][4] = acck;
    }
}

// Chunk-level parts and the final per-token gradients of key column j:
//   u_m = pair part + sum_{t>=m} dR^_t r_t gamma_t + sum_{t>m} dA^_t a_t gamma_{t-1}
//         + sum_{s<m} (dB^_s b_s + dK^_s k_s) D_{15,s} + dgamma_C gamma_C,  dw = u / w
//   da = dA^ gamma_{t-1} + F_ex pair, dr = dR^ gamma_t + F_in pair,
//   db = dB^ D_{15,t} + pair, dk = dK^ D_{15,t} + pair
template <int T0, int T1>
__device__ __forceinline__ void assemble_out(const AsmArgs &g, float (&st5)[2][5]) {
    constexpr int TK[2] = {T0, T1};
    const int j = g.j;
    const float *wcol = g.s_in + IW * 16 * LD + j;
    float wv[16], gam[16], gprev[16], dend[16], fex[16], fin[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) wv[t] = wcol[t * LD];
    {
        float gg = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) { gprev[t] = gg; gg *= wv[t]; gam[t] = gg; }
        float d = 1.f;
#pragma unroll
        for (int s = 15; s >= 0; --s) { dend[s] = d; d *= wv[s]; }
#pragma unroll
        for (int sc = 0; sc < 4; ++sc) {
            float f = 1.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * sc + e;
                fex[t] = f; f *= wv[t]; fin[t] = f;
            }
        }
    }
    const float *gA = g.s_G, *gR = g.s_G + 16 * LD, *gB = g.s_G + 32 * LD, *gK = g.s_G + 48 * LD;
    float suf[17], pre[17];
    suf[16] = 0.f;
#pragma unroll
    for (int t = 15; t >= 0; --t) {
        float x = gR[t * LD + j] * g.s_in[(IR * 16 + t) * LD + j] * gam[t];
        if (t < 15) x += gA[(t + 1) * LD + j] * g.s_in[(IA * 16 + t + 1) * LD + j] * gprev[t + 1];
        suf[t] = suf[t + 1] + x;
    }
    pre[0] = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s)
        pre[s + 1] = pre[s] + (gB[s * LD + j] * g.s_in[(IB * 16 + s) * LD + j] +
                               gK[s * LD + j] * g.s_in[(IK * 16 + s) * LD + j]) * dend[s];
    const float dgc = g.s_dgC[j] * gam[15];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int t = TK[q];
        float up = 0.f;
#pragma unroll
        for (int w8 = 0; w8 < 8; ++w8) up += g.s_U[(w8 * 16 + t) * LD + j];
        const float uval = up + suf[t] + pre[t] + dgc;
        const float dr = gR[t * LD + j] * gam[t] + fin[t] * st5[q][0];
        const float da = gA[t * LD + j] * gprev[t] + fex[t] * st5[q][2];
        const float db = gB[t * LD + j] * dend[t] + st5[q][3];
        const float dk = gK[t * LD + j] * dend[t] + st5[q][4];
        st5[q][0] = dr;
        st5[q][1] = uval / wv[t];
        st5[q][2] = da;
        st5[q][3] = db;
        st5[q][4] = dk;
    }
}

template <typename TI>
__global__ __launch_bounds__(kThreads, 1) void bwd_chunk_kernel(BwdArgs p, int32_t units) {
    extern __shared__ __align__(16) float sm[];
    // Workgroup -> (unit, group of kChunksPerGroup chunks); chunks are
    // independent given S_0 (checkpoint) and dS_C (first pass).
    const int unit = blockIdx.x % units;
    const int grp = blockIdx.x / units;
    const int H = p.seg.H;
    const int h = unit % H;
    const int sq = unit / H;
    const Unit u = resolve_unit(p.seg, sq);

    const int tid = threadIdx.x;
    const int lane0 = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // 8 waves; w and w+4 share a SIMD
    int lane = lane0, l16 = lane0 & 15, kq = lane0 >> 4;
    // The lane indices are re-derived opaquely at the start of each phase, so
    // that the many LDS addresses built from them are formed inside the phase
    // instead of being hoisted out of the chunk loop and kept live throughout.
    auto relane = [&]() {
        int lv = lane0;
        asm volatile("" : "+v"(lv));
        lane = lv; l16 = lv & 15; kq = lv >> 4;
    };
    const int w4 = wave & 3;                         // 16-row / 16-column tile of this wave
    const bool lo = wave < 4;

    float *s_in = sm + O_IN;
    float *s_Q = sm + O_Q, *s_BK = sm + O_BK, *s_AR = sm + O_AR;
    float *s_BV = sm + O_BV, *s_KV = sm + O_KV, *s_VV = sm + O_VV;
    float *s_S0 = sm + O_S0, *s_DS = sm + O_DS, *s_X = sm + O_X, *s_DR = sm + O_DR;
    float *s_G = sm + O_G, *s_M = sm + O_M, *s_gC = sm + O_GC, *s_dgC = sm + O_DGC;
    const float *sV = s_in + IV * 16 * LD, *sDY = s_in + IDY * 16 * LD;
    const float *Mlak = s_M + MLAK * 256, *Mmrb = s_M + MMRB * 256, *Mmrk = s_M + MMRK * 256;
    const float *Mw = s_M + MW * 256;

    const int64_t ts = (int64_t)H * kN;
    const int64_t base = (u.start * H + h) * kN;
    const int64_t sbase = ((int64_t)sq * H + h) * (kN * kN);

    const int it = w4;

    // Staging: element groups g = tid + 512k (k = 0, 1) of 7 streams x 16
    // tokens x 8 groups of 8; stream g >> 7 is uniform per wave.
    const int nch = (u.len + kChunk - 1) / kChunk;
    const int c_lo = grp * kChunksPerGroup;
    const int c_hi = min(nch, c_lo + kChunksPerGroup);
    if (c_lo >= c_hi) return;
    Raw<TI> raw;
    float4 ckr0, ckr1, dsr0, dsr1;              // checkpoint S_0 and dS_C of the chunk in flight
    const TI *sp[2];                            // stream of each staged group (uniform)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int st = __builtin_amdgcn_readfirstlane((tid + k * kThreads) >> 7);
        const void *vp = p.staged[st];
        sp[k] = vp ? (const TI *)vp + base : nullptr;
    }
    // Loads are issued one chunk ahead, unconditionally (token rows clamped
    // into the sequence), so the registers in flight have one definition per
    // iteration; groups of a missing stream (dy == NULL, or past the seven
    // streams) load the w row instead and stage as fill.
    const TI *wrow = (const TI *)p.w + base;
    auto issue = [&](int cc) {
        const int Lc = min(kChunk, u.len - cc * kChunk);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int g = tid + k * kThreads;
            const int t = min((g >> 3) & 15, Lc - 1), e0 = (g & 7) * 8;
            raw_load((sp[k] ? sp[k] : wrow) + (int64_t)(cc * kChunk + t) * ts + e0, raw, k);
        }
        // float4 f4 = tid + 512k of a 64x64 state: row f4 / 16, column 4 (f4 % 16)
        const int64_t so = ((u.ckpt + cc) * H + h) * (int64_t)(kN * kN) + tid * 4;
        ckr0 = *(const float4 *)(p.ckpt + so);
        ckr1 = *(const float4 *)(p.ckpt + so + kThreads * 4);
        dsr0 = *(const float4 *)(p.ws + so);
        dsr1 = *(const float4 *)(p.ws + so + kThreads * 4);
    };
    issue(c_hi - 1);

#pragma unroll 1
    for (int c = c_hi - 1; c >= c_lo; --c) {
        const int t0 = c * kChunk;
        const int L = min(kChunk, u.len - t0);
        lds_barrier();
        relane();

        // ---- stage inputs (w clamped; identity tokens past the end), the
        //      checkpoint S_0 and dS_C; then prefetch chunk c-1
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int g = tid + k * kThreads;
            if (g < 7 * 128) {
                const int st = g >> 7, t = (g >> 3) & 15, e0 = (g & 7) * 8;
                float x[8];
                if (t < L && sp[k] != nullptr) {
                    raw_unpack(raw, k, x);
                } else {
                    const float f = st == IW ? 1.f : 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = f;
                }
                if (st == IW) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = fmaxf(x[e], kMinW);
                }
                float *d = s_in + (st * 16 + t) * LD + e0;
                *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
                *(float4 *)(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
            }
        }
        {
            *(float4 *)(s_S0 + (tid >> 4) * LD + (tid & 15) * 4) = ckr0;
            *(float4 *)(s_S0 + ((tid + kThreads) >> 4) * LD + (tid & 15) * 4) = ckr1;
            *(float4 *)(s_DS + (tid >> 4) * LD + (tid & 15) * 4) = dsr0;
            *(float4 *)(s_DS + ((tid + kThreads) >> 4) * LD + (tid & 15) * 4) = dsr1;
        }
        issue(max(c - 1, c_lo));
        lds_barrier();
        relane();

        // ---- decay products and operand rows: one role per wave over the 64
        //      key columns (lane = column)
        {
            const int role = __builtin_amdgcn_readfirstlane(wave), j = lane;
            const float *w_ = s_in + IW * 16 * LD + j;
            if (role == 0) {             // A^, R^, gamma_C
                float g = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    s_Q[t * LD + j] = s_in[(IA * 16 + t) * LD + j] * g;
                    g *= w_[t * LD];
                    s_Q[(16 + t) * LD + j] = s_in[(IR * 16 + t) * LD + j] * g;
                }
                s_gC[j] = g;
            } else if (role == 1) {      // B^, K^
                float d = 1.f;
#pragma unroll
                for (int s = 15; s >= 0; --s) {
                    s_BK[s * LD + j] = s_in[(IB * 16 + s) * LD + j] * d;
                    s_BK[(16 + s) * LD + j] = s_in[(IK * 16 + s) * LD + j] * d;
                    d *= w_[s * LD];
                }
            } else if (role == 2) {      // d gamma_C[j] = sum_i dS_C[i][j] S_0[i][j]
                float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
                for (int i = 0; i < 64; i += 2) {
                    acc0 = fmaf(s_DS[i * LD + j], s_S0[i * LD + j], acc0);
                    acc1 = fmaf(s_DS[(i + 1) * LD + j], s_S0[(i + 1) * LD + j], acc1);
                }
                s_dgC[j] = acc0 + acc1;
            } else if (role == 3) {      // A' = a F_ex, R' = r F_in
#pragma unroll
                for (int sc = 0; sc < 4; ++sc) {
                    float f = 1.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 4 * sc + e;
                        s_AR[t * LD + j] = s_in[(IA * 16 + t) * LD + j] * f;
                        f *= w_[t * LD];
                        s_AR[(16 + t) * LD + j] = s_in[(IR * 16 + t) * LD + j] * f;
                    }
                }
            } else {                     // b, k, bare versions of source sub-chunk role - 4
                float wv[16], W[4];
#pragma unroll
                for (int t = 0; t < 16; ++t) wv[t] = w_[t * LD];
#pragma unroll
                for (int sc = 0; sc < 4; ++sc)
                    W[sc] = (wv[4 * sc] * wv[4 * sc + 1]) * (wv[4 * sc + 2] * wv[4 * sc + 3]);
                if (role == 4) versions<0>(wv, W, s_in, s_BV, s_KV, s_VV, j);
                else if (role == 5) versions<1>(wv, W, s_in, s_BV, s_KV, s_VV, j);
                else if (role == 6) versions<2>(wv, W, s_in, s_BV, s_KV, s_VV, j);
                else versions<3>(wv, W, s_in, s_BV, s_KV, s_VV, j);
            }
        }
        lds_barrier();
        relane();

        // ---- waves 0-3: P_a = A^ S_0^T (value rows 16*w4..). waves 4-7: the
        //      four 16x16 matrices on VALU (one pair of dots per thread) and, on
        //      MFMA, dR^ = dY S_0 and dK^ = V dS_C for key columns 16*w4..
        f32x4 pa = {0.f, 0.f, 0.f, 0.f};
        if (lo) {
            pa = mm_AtBt(pa, s_Q, LD, s_S0 + 16 * it * LD, LD, l16, kq, 64);
        } else {
            const int jc = 16 * w4;
            f32x4 g1 = {0.f, 0.f, 0.f, 0.f}, g3 = g1;
            g1 = mm_AtB(g1, sDY, LD, s_S0 + jc, LD, l16, kq, 64);
            g3 = mm_AtB(g3, sV, LD, s_DS + jc, LD, l16, kq, 64);
            const int item = tid - 256;
            int t, s, mat;
            if (item < 120) {
                t = 1;
                while ((t + 1) * t / 2 <= item) ++t;
                s = item - t * (t - 1) / 2;
                mat = 0;
            } else {
                const int mi = item - 120;
                t = 0;
                while ((t + 1) * (t + 2) / 2 <= mi) ++t;
                s = mi - t * (t + 1) / 2;
                mat = 1;
            }
            const int vrow = ver_off(t >> 2) + s;
            const float *ar = s_AR + (16 * mat + t) * LD;
            const float *bv = s_BV + vrow * LD;
            const float *kv = s_KV + vrow * LD;
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
            s_M[(2 * mat) * 256 + t * 16 + s] = db0 + db1;
            s_M[(2 * mat + 1) * 256 + t * 16 + s] = dk0 + dk1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = 4 * kq + r;
                s_G[(1 * 16 + tt) * LD + jc + l16] = g1[r];
                s_G[(3 * 16 + tt) * LD + jc + l16] = g3[r];
            }
        }
        lds_barrier();
        relane();

        // ---- W = (I - L_ab)^-1 (wave 0, 16 lanes); upper parts cleared (wave 1);
        //      dM_rk = dY V^T (wave 2; lower part incl. the diagonal)
        if (wave == 0) {
            if (lane < 16) {
                float x[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) x[t] = t == lane ? 1.f : 0.f;
#pragma unroll
                for (int s2 = 0; s2 < 15; ++s2) {
#pragma unroll
                    for (int t = s2 + 1; t < 16; ++t) x[t] = fmaf(s_M[MLAB * 256 + t * 16 + s2], x[s2], x[t]);
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) s_M[MW * 256 + t * 16 + lane] = x[t];
            }
        } else if (wave == 1) {
            const int m = lane >> 4, row = lane & 15;
            const int first = m < 2 ? row : row + 1;
            for (int c2 = first; c2 < 16; ++c2) s_M[m * 256 + row * 16 + c2] = 0.f;
        } else if (wave == 2) {
            f32x4 gm = {0.f, 0.f, 0.f, 0.f};
            gm = mm_AtBt(gm, sDY, LD, sV, LD, l16, kq, 64);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * kq + r;
                s_M[MDMRK * 256 + t * 16 + l16] = l16 <= t ? gm[r] : 0.f;
            }
        }
        lds_barrier();
        relane();

        // ---- value side. waves 0-3 (rows 16*w4..): X = W (P_a + L_ak V);
        //      dX = B^ dS_C^T + M_rb^T dY; drhs = W^T dX.
        //      waves 4-7 (same rows): dV partial = K^ dS_C^T + M_rk^T dY
        const int i0 = 16 * it;
        f32x4 dvp = {0.f, 0.f, 0.f, 0.f};
        if (lo) {
            const f32x4 rhs = mm_AtB(pa, Mlak, 16, sV + i0, LD, l16, kq, 16);
            f32x4 xx = {0.f, 0.f, 0.f, 0.f};
            {
                const float4 wr = *(const float4 *)(Mw + l16 * 16 + 4 * kq);
                xx = mfma4(wr.x, rhs[0], xx); xx = mfma4(wr.y, rhs[1], xx);
                xx = mfma4(wr.z, rhs[2], xx); xx = mfma4(wr.w, rhs[3], xx);
            }
            f32x4 dx = {0.f, 0.f, 0.f, 0.f};
            dx = mm_AtBt(dx, s_BK, LD, s_DS + i0 * LD, LD, l16, kq, 64);
            dx = mm_TB(dx, Mmrb, 16, sDY + i0, LD, l16, kq);
            f32x4 dr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) dr = mfma4(Mw[(4 * kq + e) * 16 + l16], dx[e], dr);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * kq + r;
                s_X[t * LD + i0 + l16] = xx[r];
                s_DR[t * LD + i0 + l16] = dr[r];
            }
        } else {
            dvp = mm_AtBt(dvp, s_BK + 16 * LD, LD, s_DS + i0 * LD, LD, l16, kq, 64);
            dvp = mm_TB(dvp, Mmrk, 16, sDY + i0, LD, l16, kq);
        }
        lds_barrier();
        relane();

        // ---- key side and the state gradient:
        //      waves 4-7 finish dV = partial + L_ak^T drhs and store it;
        //      waves 0-3: dA^ = drhs S_0, waves 4-7: dB^ = X dS_C (key columns 16*w4..);
        //      waves 0, 1, 2: dL_ab = drhs X^T, dL_ak = drhs V^T, dM_rb = dY X^T;
        //      every wave: its two dS_0^T tiles
        {
            const int jc = 16 * w4;
            if (!lo) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = 4 * kq + e;
                    dvp = mfma4(Mlak[k * 16 + l16], s_DR[k * LD + i0 + l16], dvp);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * kq + r;
                    if (t < L) IO<TI>::st((TI *)p.dv, base + (int64_t)(t0 + t) * ts + i0 + l16, dvp[r]);
                }
                f32x4 g2 = {0.f, 0.f, 0.f, 0.f};
                g2 = mm_AtB(g2, s_X, LD, s_DS + jc, LD, l16, kq, 64);
#pragma unroll
                for (int r = 0; r < 4; ++r) s_G[(2 * 16 + 4 * kq + r) * LD + jc + l16] = g2[r];
            } else {
                f32x4 g0 = {0.f, 0.f, 0.f, 0.f};
                g0 = mm_AtB(g0, s_DR, LD, s_S0 + jc, LD, l16, kq, 64);
#pragma unroll
                for (int r = 0; r < 4; ++r) s_G[(0 * 16 + 4 * kq + r) * LD + jc + l16] = g0[r];
                if (wave < 3) {
                    const float *lhs = wave < 2 ? s_DR : sDY;
                    const float *rt = wave == 1 ? sV : s_X;
                    f32x4 gm = {0.f, 0.f, 0.f, 0.f};
                    gm = mm_AtBt(gm, lhs, LD, rt, LD, l16, kq, 64);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 4 * kq + r;
                        const bool keep = wave < 2 ? (l16 < t) : (l16 <= t);
                        s_M[(MDLAB + wave) * 256 + t * 16 + l16] = keep ? gm[r] : 0.f;
                    }
                }
            }
        }
        lds_barrier();
        relane();

        // ---- key-side gradient assembly: wave w owns tokens {w, 15-w} of every
        //      key column (lane = column); u's pair part is summed over the 8 waves
        {
            const int j = lane;
            AsmArgs aa{s_in, s_AR, s_BV, s_KV, s_VV, s_G, s_M, s_dgC, s_S0, j, wave};
            float st5[2][5];
            switch (__builtin_amdgcn_readfirstlane(wave)) {
            case 0: assemble_rows<0, 15>(aa, st5); break;
            case 1: assemble_rows<1, 14>(aa, st5); break;
            case 2: assemble_rows<2, 13>(aa, st5); break;
            case 3: assemble_rows<3, 12>(aa, st5); break;
            case 4: assemble_rows<4, 11>(aa, st5); break;
            case 5: assemble_rows<5, 10>(aa, st5); break;
            case 6: assemble_rows<6, 9>(aa, st5); break;
            default: assemble_rows<7, 8>(aa, st5); break;
            }
            lds_barrier();
            relane();
            switch (__builtin_amdgcn_readfirstlane(wave)) {
            case 0: assemble_out<0, 15>(aa, st5); break;
            case 1: assemble_out<1, 14>(aa, st5); break;
            case 2: assemble_out<2, 13>(aa, st5); break;
            case 3: assemble_out<3, 12>(aa, st5); break;
            case 4: assemble_out<4, 11>(aa, st5); break;
            case 5: assemble_out<5, 10>(aa, st5); break;
            case 6: assemble_out<6, 9>(aa, st5); break;
            default: assemble_out<7, 8>(aa, st5); break;
            }
            const int tks[2] = {wave, 15 - wave};
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int t = tks[q];
                if (t < L) {
                    const int64_t o = base + (int64_t)(t0 + t) * ts + j;
                    IO<TI>::st((TI *)p.dr, o, st5[q][0]);
                    IO<TI>::st((TI *)p.dw, o, st5[q][1]);
                    IO<TI>::st((TI *)p.da, o, st5[q][2]);
                    IO<TI>::st((TI *)p.db, o, st5[q][3]);
                    IO<TI>::st((TI *)p.dk, o, st5[q][4]);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_backward(const BwdArgs &args, hipStream_t stream) {
    BwdArgs a = args;
    const void *staged[8] = {a.r, a.w, a.k, a.a, a.b, a.v, a.dy, nullptr};
    static_assert(IR == 0 && IW == 1 && IK == 2 && IA == 3 && IB == 4 && IV == 5 && IDY == 6,
                  "staged stream order");
    for (int i = 0; i < 8; ++i) a.staged[i] = staged[i];
    const int S = a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B;
    const int32_t units = S * a.seg.H;
    const size_t lds = (size_t)LDS_FLOATS * sizeof(float);
    auto fn = a.dtype == 1 ? bwd_chunk_kernel<uint16_t> : bwd_chunk_kernel<float>;
    hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // A sequence lies within one row of T tokens, so it has at most ceil(T / 16) chunks.
    const int max_chunks = (a.seg.T + kChunk - 1) / kChunk;
    const int64_t groups = (max_chunks + kChunksPerGroup - 1) / kChunksPerGroup;
    hipLaunchKernelGGL(fn, dim3((unsigned)(groups * units)), dim3(kThreads), lds, stream, a, units);
    return hipGetLastError();
}

}  // namespace wkv7
