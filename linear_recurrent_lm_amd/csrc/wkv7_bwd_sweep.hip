// WKV-7 backward, first pass: the state-gradient sweep.
//
// With the chunk form of the forward (tokens t = 0..15 of a chunk, entering
// state S_0, leaving state S_C)
//     X = W (A^ S_0^T + L_ak V),  W = (I - L_ab)^-1
//     Y = R^ S_0^T + M_rb X + M_rk V
//     S_C = S_0 diag(gamma_C) + X^T B^ + V^T K^
// the gradient of the state entering a chunk follows from the gradient of
// the state leaving it without any reference to the state itself:
//     dX   = B^ dS_C^T + M_rb^T dY,     drhs = W^T dX
//     dS_0 = dS_C diag(gamma_C) + drhs^T A^ + dY^T R^
// (rows A^_t = gamma_{t-1} a_t, R^_t = gamma_t r_t, B^_s = D_{15,s} b_s). This
// kernel runs that recurrence from the last chunk to the first and stores
// dS_C of every chunk in the workspace (one 64x64 fp32 slot per checkpoint
// slot), plus dS_0 of the first chunk as the initial-state gradient. The
// per-chunk gradients of r, w, k, v, a, b then no longer depend on each
// other and are computed in parallel by the second pass.
//
// The structure mirrors the forward kernel: state waves hold 16 value rows x
// 64/KS columns of dS^T in MFMA accumulators (lane l: dS[row0 + l%16][16*jt +
// 4*(l/16) + r]); with KS = 2 the two waves sharing 16 rows hold one half of
// the key columns each and add each other's partial dX (a sum over keys)
// through LDS, so the serial chain spreads over four SIMDs when a workgroup
// holds only 32 rows. Eight operand waves build, one chunk ahead, the rows B^,
// A^, R^, gamma_C, dY and the 16x16 matrices M_rb and W (L_ab only feeds W),
// with the same split-point products and within-sub-chunk dot products, into
// a double-buffered LDS hand-off; two workgroup barriers per chunk. The
// decay is clamped to w >= 2^-30 throughout, as in the second pass. The
// products run on FP32 MFMA, except that with bf16 streams the two against
// dy (whose values are exact in bf16) take their other operand in three bf16
// pieces on bf16 MFMA.
#include <type_traits>

#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr int kPrepWaves = 8;
constexpr int QLD = 68;    // row stride (floats) of 64-wide rows
constexpr int KLD = 36;    // row stride of the transposed [A^|R^] tile
constexpr int VLD = 20;    // row stride of the transposed dY tile
constexpr int MLD = 20;    // row stride of the 16x16 matrices
constexpr float kMinW = 9.313225746154785e-10f;   // 2^-30

// staged streams
enum { SR = 0, SW, SA, SB, SDY, kStreams };
enum { MMRBT = 0, MWT };

// acc += sum over 16 indices of a[e] y[e] (this lane's 4 of them), a fp32 in
// three bf16 pieces (24 bits) and y holding bf16 values (dy of bf16 streams):
// two K = 32 bf16 MFMAs, which leave the SIMD's VALU free where the four
// FP32 ones held it
__device__ __forceinline__ f32x4 mm_k16_3x(f32x4 acc, float4 a, float4 y) {
    uint32_t h0, m0, l0, h1, m1, l1;
    split3(a.x, a.y, h0, m0, l0);
    split3(a.z, a.w, h1, m1, l1);
    const uint32_t y0 = pk_bf16(y.x, y.y), y1 = pk_bf16(y.z, y.w);
    acc = mfma_bf16_k32(u32x4_t{l0, l1, 0u, 0u}, u32x4_t{y0, y1, 0u, 0u}, acc);
    return mfma_bf16_k32(u32x4_t{h0, h1, m0, m1}, u32x4_t{y0, y1, y0, y1}, acc);
}

namespace lay {
constexpr int IN = 0;                       // [2][5][16][64] r w a b dy, by chunk parity
constexpr int IN_SIZE = kStreams * 16 * 64;
constexpr int AR = IN + 2 * IN_SIZE;        // [32][QLD] A'_t = a_t F_ex(t), R'_t = r_t F_in(t)
constexpr int AWR = AR + 32 * QLD;          // [8][QLD]  A'_t W_2, R'_t W_2 for t = 12..15
constexpr int BD = AWR + 8 * QLD;           // [16][QLD] b_s / F_s
constexpr int BL = BD + 16 * QLD;           // [32][QLD] b rows scaled to the split points (k rows unused)
constexpr int LAB = BL + 32 * QLD;          // [16][MLD] L_ab (upper part stays zero)
constexpr int BUF = LAB + 16 * MLD;
// within a hand-off buffer
constexpr int B_BH = 0;                     // [16][QLD] B^ rows
constexpr int B_ART = B_BH + 16 * QLD;      // [64][KLD] A^ | R^ by key column j
constexpr int B_DYT = B_ART + 64 * KLD;     // [64][VLD] dY by value row i
constexpr int B_M = B_DYT + 64 * VLD;       // [2][16][MLD] M_rb^T, W^T
constexpr int B_GC = B_M + 2 * 16 * MLD;    // [64] gamma_C
constexpr int BUF_SIZE = B_GC + 64;
constexpr int XCH = BUF + 2 * BUF_SIZE;     // [4 waves][64 lanes][4] partial dX (key split)
constexpr int TOTAL = XCH + 4 * 256;
static_assert(BUF % 4 == 0 && BUF_SIZE % 4 == 0 && IN_SIZE % 4 == 0, "16-byte aligned buffers");
}  // namespace lay

// HB: dS_C and drhs go to the workspace in bf16 (bf16 streams with bf16
// gradients, whose second pass rounds every operand to one bf16 piece)
template <typename TI, int NMW, int KS, bool HB>
__global__ __launch_bounds__(64 * (NMW + kPrepWaves), 1) void dsweep_kernel(BwdArgs p, int32_t units) {
    constexpr int NG = NMW / KS;       // 16-row groups per workgroup
    constexpr int RB = 16 * NG;        // value rows per workgroup
    constexpr int NRB = 64 / RB;       // row blocks per unit
    constexpr int NQ = 4 / KS;         // 16-column key tiles per state wave
    static_assert(KS == 1 || KS == 2, "key split of 1 or 2");
    // bf16 streams: the products against dy (exact in bf16) take the other
    // operand in three bf16 pieces on bf16 MFMA
    constexpr bool kX3 = std::is_same<TI, uint16_t>::value;
    extern __shared__ __align__(16) float sm[];

    int unit, rb;
    if (NRB == 1) {
        unit = blockIdx.x;
        rb = 0;
    } else {               // row blocks of one unit on one XCD (shared L2)
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15, kq = lane >> 4;
    const int64_t ts = (int64_t)H * kN;
    const int64_t base = (u.start * H + h) * kN;
    const int64_t sbase = ((int64_t)sq * H + h) * (kN * kN);
    const int nch = (u.len + kChunk - 1) / kChunk;

    if (wave < NMW) {
        // ================= state waves =================
        const int rg = wave % NG, kh = wave / NG;        // row group, key part
        const int irow = i0 + 16 * rg + l16;             // value row of this lane
        const int q0 = kh * NQ;                          // first key tile of this wave
        f32x4 acc[NQ];                                   // dS^T tiles
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
            if (p.ds_out) {
                const float4 v4 = *(const float4 *)(p.ds_out + sbase + (int64_t)irow * kN + 16 * (q0 + qq) + 4 * kq);
                acc[qq] = f32x4{v4.x, v4.y, v4.z, v4.w};
            } else {
                acc[qq] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        float *xch_own = sm + lay::XCH + wave * 256 + lane * 4;
        const float *xch_mate = sm + lay::XCH + (rg + (1 - kh) * NG) * 256 + lane * 4;
        // Iteration k advances chunk cs = nch - k (built in iteration k - 1).
#pragma unroll 1
        for (int k = 0; k <= nch; ++k) {
            const int cs = nch - k;
            const float *buf = sm + lay::BUF + (cs & 1) * lay::BUF_SIZE;
            f32x4 dx = {0.f, 0.f, 0.f, 0.f};
            lds_barrier();
            // ---- phase X (W of this chunk is being solved meanwhile): store dS_C;
            //      dX = B^ dS_C^T (over this wave's key columns) + M_rb^T dY (one
            //      key part when split); dS^T = diag(gamma) dS^T + R^^T dY
            if (k >= 1) {
                const int64_t wo = ((u.ckpt + cs) * H + h) * (int64_t)(kN * kN) + (int64_t)irow * kN;
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq) {
                    const int64_t o = wo + 16 * (q0 + qq) + 4 * kq;
                    if constexpr (HB) {
                        *(uint2 *)((uint16_t *)p.ws + o) =
                            make_uint2(pk_bf16(acc[qq][0], acc[qq][1]), pk_bf16(acc[qq][2], acc[qq][3]));
                    } else {
                        *(float4 *)(p.ws + o) = make_float4(acc[qq][0], acc[qq][1], acc[qq][2], acc[qq][3]);
                    }
                }
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq) {
                    const int q = q0 + qq;
                    const float4 b4 = *(const float4 *)(buf + lay::B_BH + l16 * QLD + 16 * q + 4 * kq);
                    dx = mfma4(b4.x, acc[qq][0], dx);
                    dx = mfma4(b4.y, acc[qq][1], dx);
                    dx = mfma4(b4.z, acc[qq][2], dx);
                    dx = mfma4(b4.w, acc[qq][3], dx);
                }
                const float4 dyb = *(const float4 *)(buf + lay::B_DYT + irow * VLD + 4 * kq);
                if (KS == 1 || kh == 0) {
                    const float4 mrbt = *(const float4 *)(buf + lay::B_M + MMRBT * 16 * MLD + l16 * MLD + 4 * kq);
                    if constexpr (kX3) {
                        dx = mm_k16_3x(dx, mrbt, dyb);
                    } else {
                        dx = mfma4(mrbt.x, dyb.x, dx); dx = mfma4(mrbt.y, dyb.y, dx);
                        dx = mfma4(mrbt.z, dyb.z, dx); dx = mfma4(mrbt.w, dyb.w, dx);
                    }
                }
                if (KS > 1) *(float4 *)xch_own = make_float4(dx[0], dx[1], dx[2], dx[3]);
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq) {
                    const int q = q0 + qq;
                    const float4 g4 = *(const float4 *)(buf + lay::B_GC + 16 * q + 4 * kq);
                    const float4 r4 = *(const float4 *)(buf + lay::B_ART + (16 * q + l16) * KLD + 16 + 4 * kq);
                    f32x4 a = acc[qq];
                    a[0] *= g4.x; a[1] *= g4.y; a[2] *= g4.z; a[3] *= g4.w;
                    if constexpr (kX3) {
                        a = mm_k16_3x(a, r4, dyb);
                    } else {
                        a = mfma4(r4.x, dyb.x, a); a = mfma4(r4.y, dyb.y, a);
                        a = mfma4(r4.z, dyb.z, a); a = mfma4(r4.w, dyb.w, a);
                    }
                    acc[qq] = a;
                }
            }
            lds_barrier();
            // ---- phase Y: (add the partner's partial dX); drhs = W^T dX;
            //      dS^T += A^^T drhs
            if (k >= 1) {
                if (KS > 1) {
                    const float4 pd = *(const float4 *)xch_mate;
                    dx[0] += pd.x; dx[1] += pd.y; dx[2] += pd.z; dx[3] += pd.w;
                }
                const float4 wt = *(const float4 *)(buf + lay::B_M + MWT * 16 * MLD + l16 * MLD + 4 * kq);
                f32x4 dr = {0.f, 0.f, 0.f, 0.f};
                dr = mfma4(wt.x, dx[0], dr); dr = mfma4(wt.y, dx[1], dr);
                dr = mfma4(wt.z, dx[2], dr); dr = mfma4(wt.w, dx[3], dr);
                if (KS == 1 || kh == 0) {        // drhs[t][i] of this chunk for the second pass
                    const int64_t dof = ((u.ckpt + cs) * H + h) * (int64_t)(kChunk * kN) + irow;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (HB) ((uint16_t *)p.ws_dr)[dof + (4 * kq + r) * kN] = f32_to_bf16(dr[r]);
                        else p.ws_dr[dof + (4 * kq + r) * kN] = dr[r];
                    }
                }
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq) {
                    const int q = q0 + qq;
                    const float4 a4 = *(const float4 *)(buf + lay::B_ART + (16 * q + l16) * KLD + 4 * kq);
                    f32x4 a = acc[qq];
                    a = mfma4(a4.x, dr[0], a); a = mfma4(a4.y, dr[1], a);
                    a = mfma4(a4.z, dr[2], a); a = mfma4(a4.w, dr[3], a);
                    acc[qq] = a;
                }
            }
        }
        if (p.ds0) {
            float *op = p.ds0 + sbase + (int64_t)irow * kN;
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq)
                *(float4 *)(op + 16 * (q0 + qq) + 4 * kq) = make_float4(acc[qq][0], acc[qq][1], acc[qq][2], acc[qq][3]);
        }
        return;
    }

    // ================= operand waves =================
    const int pw = wave - NMW;                 // 0..7, uniform
    const int ptid = tid - 64 * NMW;           // 0..511
    const int sid = ptid - 256;                // staging thread index (operand waves 4..7)
    float *s_AR = sm + lay::AR;
    float *s_AWR = sm + lay::AWR;
    float *s_BD = sm + lay::BD;
    float *s_BL = sm + lay::BL;
    float *s_Lab = sm + lay::LAB;

    // Staging (operand waves 4-7): element group g = sid + 256k (k = 0..2) of
    // 5 streams x 16 tokens x 8 groups of 8 elements (groups 640.. unused);
    // stream g >> 7 is uniform per wave. Loads are issued ahead,
    // unconditionally (chunk index and token rows clamped into the sequence;
    // a missing dy stages as zeros), so the registers in flight have exactly
    // one definition per iteration. For 16-bit inputs two register sets
    // alternate, which keeps each chunk's loads in flight for two chunk
    // periods (HBM latency under load exceeds one).
    constexpr bool kTwoSets = sizeof(TI) == 2;
    Raw<TI, 3> raw, raw1;
    const TI *sp[3];
    bool sv[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int st = __builtin_amdgcn_readfirstlane((sid + 256 * k) >> 7);
        const void *vp = st == SR ? p.r : st == SW ? p.w : st == SA ? p.a : st == SB ? p.b
                       : (st == SDY && p.dy) ? p.dy : p.w;
        sp[k] = (const TI *)vp + base;
        sv[k] = st < SDY || (st == SDY && p.dy != nullptr);
    }
    auto issue = [&](int cc, Raw<TI, 3> &raw) {     // 0 <= cc < nch
        const int Lc = min(kChunk, u.len - cc * kChunk);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int g = sid + 256 * k;
            const int t = min((g >> 3) & 15, Lc - 1), e0 = (g & 7) * 8;
            raw_load(sp[k] + (int64_t)(cc * kChunk) * ts + row_off(t, ts, e0), raw, k);
        }
    };
    auto stage = [&](int cc, const Raw<TI, 3> &raw) {
        const int Lc = min(kChunk, u.len - cc * kChunk);
        float *s_in = sm + lay::IN + (cc & 1) * lay::IN_SIZE;
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int g = sid + 256 * k;
            const int st = g >> 7, t = (g >> 3) & 15, e0 = (g & 7) * 8;
            if (st >= kStreams) continue;
            float x[8];
            if (t < Lc && sv[k]) {
                raw_unpack(raw, k, x);
                if (st == SW) {
                    decay_of<8>(x, p.logw);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = fmaxf(x[e], kMinW);
                }
            } else {                           // identity tokens past the end
                const float f = st == SW ? 1.f : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = f;
            }
            float *d = s_in + (st * 16 + t) * 64 + e0;
            *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
            *(float4 *)(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
        }
    };

    // ---- phase X (operand waves 1-3): rows the 16x16 matrices are built from:
    //      A' = a F_ex (wave 1), R' = r F_in (wave 2), b rows (wave 3)
    auto matrix_rows = [&](const float *s_in) {
        const int j = lane;
        const int role = pw - 1;
        const int st = role == 0 ? SA : role == 1 ? SR : SB;
        float wv[16], xv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            wv[t] = s_in[SW * 1024 + t * 64 + j];
            xv[t] = s_in[st * 1024 + t * 64 + j];
        }
        if (role < 2) {            // times W_2 for t >= 12 as well
            const int inc = role;
            float o[16];
#pragma unroll
            for (int sc = 0; sc < 4; ++sc) {
                float f = 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * sc + e;
                    if (inc) f *= wv[t];
                    o[t] = xv[t] * f;
                    if (!inc) f *= wv[t];
                }
            }
            const float W2 = (wv[8] * wv[9]) * (wv[10] * wv[11]);
#pragma unroll
            for (int t = 0; t < 16; ++t) s_AR[(16 * inc + t) * QLD + j] = o[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) s_AWR[(4 * inc + e) * QLD + j] = o[12 + e] * W2;
        } else {                   // b_s / F_s, and b_s scaled to the split points
            float od[16], os[12];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float suf = 1.f;                 // suf = prod_{s<u<4q+4} w_u, built downwards
#pragma unroll
                for (int e = 3; e >= 0; --e) {
                    if (q < 3) os[4 * q + e] = xv[4 * q + e] * suf;
                    suf *= wv[4 * q + e];
                }
                // 1 / F_s from one reciprocal of the sub-chunk's product F_{4q+3},
                // then 1 / F_{s-1} = w_s / F_s going down
                float inv = __builtin_amdgcn_rcpf(suf);
#pragma unroll
                for (int e = 3; e >= 0; --e) {
                    od[4 * q + e] = xv[4 * q + e] * inv;
                    inv *= wv[4 * q + e];
                }
            }
            const float W1 = (wv[4] * wv[5]) * (wv[6] * wv[7]);
#pragma unroll
            for (int s = 0; s < 16; ++s) s_BD[s * QLD + j] = od[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s_BL[e * QLD + j] = os[e] * W1;              // s = e scaled to 8
                s_BL[(16 + e) * QLD + j] = os[e];            // s = e scaled to 4
                s_BL[(4 + e) * QLD + j] = os[4 + e];         // s = 4+e scaled to 8
                s_BL[(24 + e) * QLD + j] = os[8 + e];        // s = 8+e scaled to 12
            }
        }
    };

    // ---- phase Y (operand waves 6, 7): hand-off rows for the state waves:
    //      B^ rows, gamma_C and dY by value row (wave 6); A^, R^ by key column (wave 7)
    auto handoff_rows = [&](const float *s_in, float *buf) {
        const int j = lane;
        float wv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) wv[t] = s_in[SW * 1024 + t * 64 + j];
        if (pw == 6) {
            float bv[16], dv[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                bv[t] = s_in[SB * 1024 + t * 64 + j];
                dv[t] = s_in[SDY * 1024 + t * 64 + j];
            }
            float d = 1.f;
#pragma unroll
            for (int s = 15; s >= 0; --s) { bv[s] *= d; d *= wv[s]; }
#pragma unroll
            for (int s = 0; s < 16; ++s) buf[lay::B_BH + s * QLD + j] = bv[s];
            buf[lay::B_GC + j] = d;
#pragma unroll
            for (int t = 0; t < 16; t += 4)
                *(float4 *)(buf + lay::B_DYT + j * VLD + t) = make_float4(dv[t], dv[t + 1], dv[t + 2], dv[t + 3]);
        } else {
            float av[16], rv[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                av[t] = s_in[SA * 1024 + t * 64 + j];
                rv[t] = s_in[SR * 1024 + t * 64 + j];
            }
            float g = 1.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                av[t] *= g;
                g *= wv[t];
                rv[t] *= g;
            }
            float *dst = buf + lay::B_ART + j * KLD;
#pragma unroll
            for (int t = 0; t < 16; t += 4) {
                *(float4 *)(dst + t) = make_float4(av[t], av[t + 1], av[t + 2], av[t + 3]);
                *(float4 *)(dst + 16 + t) = make_float4(rv[t], rv[t + 1], rv[t + 2], rv[t + 3]);
            }
        }
    };

    // ---- phase Y (operand waves 0-3): L_ab (into s_Lab) and M_rb^T. Waves 0, 1:
    //      the cross-sub-chunk blocks on MFMA (b columns only); waves 2, 3: the
    //      within-sub-chunk pairs on VALU
    auto matrices = [&](float *buf) {
        float *mrbt = buf + lay::B_M + MMRBT * 16 * MLD;
        if (pw < 2) {
            // wave 0: split at 8: rows m < 8 are a rows t = 8+m, m >= 8 r rows t = m;
            //         columns n < 8 are b rows s = n (n >= 8: k rows, unused here).
            // wave 1: splits at 4 and 12: m < 8 covers t in 4..7, m >= 8 t in 12..15
            //         (a rows where m & 4 == 0); n likewise for s in 0..3 and 8..11.
            const int m = l16;
            const float *arow, *brow;
            if (pw == 0) {
                arow = m < 4 ? s_AR + (8 + m) * QLD : m < 8 ? s_AWR + (m - 4) * QLD
                     : m < 12 ? s_AR + (16 + m) * QLD : s_AWR + (m - 8) * QLD;
                brow = s_BL + l16 * QLD;
            } else {
                arow = s_AR + ((m & 4) ? 16 + m : 4 + m) * QLD;
                brow = s_BL + (16 + l16) * QLD;
            }
            const f32x4 d = rows_product(arow, brow, kq);
            const int n = l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int mm = 4 * kq + r;
                bool isA, isB, valid = true;
                int t, s;
                if (pw == 0) {
                    isA = mm < 8; t = isA ? 8 + mm : mm;
                    isB = n < 8;  s = n;
                } else {
                    isA = (mm & 4) == 0; t = isA ? 4 + mm : mm;
                    isB = (n & 4) == 0;  s = n;
                    valid = (mm < 8) == (n < 8);
                }
                if (valid && isB) {
                    if (isA) s_Lab[t * MLD + s] = d[r];
                    else mrbt[s * MLD + t] = d[r];
                }
            }
        } else {
            // 64 items (sub-chunk p, pair k) x 4 quarters of the 64 columns = 256
            // units, two per lane of waves 2 and 3
            float db[2];
            int tt[2], ss[2];
            bool lt[2];
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int unit_ = ptid - 128 + 128 * v;
                const int item = unit_ >> 2, qtr = unit_ & 3;
                const int sc = item >> 4, kk = item & 15;
                int et, es;
                const bool isL = kk < 6;
                if (isL) {                 // s < t
                    et = 1 + (kk >= 1) + (kk >= 3);
                    es = kk - et * (et - 1) / 2;
                } else {                   // s <= t
                    const int mi = kk - 6;
                    et = (mi >= 1) + (mi >= 3) + (mi >= 6);
                    es = mi - et * (et + 1) / 2;
                }
                const int t = 4 * sc + et, s = 4 * sc + es;
                const float *ar = s_AR + ((isL ? 0 : 16) + t) * QLD + 16 * qtr;
                const float *bd = s_BD + s * QLD + 16 * qtr;
                float b_ = 0.f;
#pragma unroll
                for (int jj = 0; jj < 16; jj += 4) {
                    const float4 x = *(const float4 *)(ar + jj);
                    const float4 b = *(const float4 *)(bd + jj);
                    b_ = fmaf(x.x, b.x, b_); b_ = fmaf(x.y, b.y, b_);
                    b_ = fmaf(x.z, b.z, b_); b_ = fmaf(x.w, b.w, b_);
                }
                db[v] = b_; tt[v] = t; ss[v] = s; lt[v] = isL;
            }
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const float b_ = quad_sum(db[v]);
                if ((lane & 3) == 0) {
                    if (lt[v]) s_Lab[tt[v] * MLD + ss[v]] = b_;
                    else mrbt[ss[v] * MLD + tt[v]] = b_;
                }
            }
        }
    };

    // ---- W^T = ((I - L_ab)^-1)^T (phase X, wave 0: column c = lane / 4 of W,
    //      rows t = lane % 4 + 4i held by the 4 lanes of a quad, forward
    //      substitution); W of chunk cw also goes to the workspace for the
    //      second pass (from the first row block of the unit only)
    auto solve_w = [&](float *buf, int cw) {
        const int col = lane >> 2, q = lane & 3;
        float Lr[4][16], x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int s = 0; s < 16; s += 4) {
                const float4 v = *(const float4 *)(s_Lab + (q + 4 * i) * MLD + s);
                Lr[i][s] = v.x; Lr[i][s + 1] = v.y; Lr[i][s + 2] = v.z; Lr[i][s + 3] = v.w;
            }
            x[i] = q + 4 * i == col ? 1.f : 0.f;
        }
#pragma unroll
        for (int s = 0; s < 15; ++s) {
            const float xs = quad_bcast(x[s >> 2], s & 3);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float nx = fmaf(Lr[i][s], xs, x[i]);
                x[i] = q + 4 * i > s ? nx : x[i];
            }
        }
        // W^T[col][t] = W[t][col]: the quad's four lanes hold t = q + 4i
#pragma unroll
        for (int i = 0; i < 4; ++i) buf[lay::B_M + MWT * 16 * MLD + col * MLD + q + 4 * i] = x[i];
        if (rb == 0) {
            float *wp = p.ws_w + ((u.ckpt + cw) * H + h) * (int64_t)(kChunk * kChunk) + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) wp[(q + 4 * i) * kChunk] = x[i];
        }
    };

    // Entries of L_ab and of the hand-off matrices that are never written
    // (upper parts) stay zero.
    for (int q = ptid; q < 16 * MLD + 2 * lay::BUF_SIZE; q += 64 * kPrepWaves) sm[lay::LAB + q] = 0.f;
    if (nch == 0) {            // nothing to build; match the state waves' two barriers
        lds_barrier();
        lds_barrier();
        return;
    }

    // Iteration k builds chunk cp = nch - 1 - k (phase X: matrix rows, W of
    // chunk cp + 1, staging of chunk cp - 1; phase Y: the 16x16 matrices and
    // the hand-off rows of chunk cp). The state waves need W only in phase Y.
    if (pw >= 4) {
        // iteration k stages chunk cp - 1 from set rw and refills rw with
        // chunk cp - 1 - d (d = 2 with two sets, else 1)
        auto step = [&](int k, Raw<TI, 3> &rw, int d) {
            const int cp = nch - 1 - k;
            float *buf = sm + lay::BUF + (cp & 1) * lay::BUF_SIZE;
            const float *s_in = sm + lay::IN + (cp & 1) * lay::IN_SIZE;
            lds_barrier();
            if (cp >= 1) stage(cp - 1, rw);
            issue(max(cp - 1 - d, 0), rw);
            lds_barrier();
            if (cp >= 0 && pw >= 6) handoff_rows(s_in, buf);
        };
        issue(nch - 1, raw);
        stage(nch - 1, raw);
        if constexpr (kTwoSets) {
            issue(max(nch - 2, 0), raw1);
            // keep every load of chunk nch-2 ahead of chunk nch-3's, so that
            // staging chunk nch-2 waits for its own loads only
            __builtin_amdgcn_sched_barrier(0);
            issue(max(nch - 3, 0), raw);
#pragma unroll 1
            for (int k = 0; k <= nch; k += 2) {
                step(k, raw1, 2);                  // chunk nch-2-k was loaded into raw1
                if (k + 1 > nch) break;
                step(k + 1, raw, 2);               // chunk nch-3-k was loaded into raw
            }
        } else {
            issue(max(nch - 2, 0), raw);
#pragma unroll 1
            for (int k = 0; k <= nch; ++k) step(k, raw, 1);
        }
    } else {
#pragma unroll 1
        for (int k = 0; k <= nch; ++k) {
            const int cp = nch - 1 - k;
            float *buf = sm + lay::BUF + (cp & 1) * lay::BUF_SIZE;
            const float *s_in = sm + lay::IN + (cp & 1) * lay::IN_SIZE;
            lds_barrier();
            if (pw == 0) {
                if (k >= 1) solve_w(sm + lay::BUF + ((cp + 1) & 1) * lay::BUF_SIZE, cp + 1);
            } else if (cp >= 0) {
                matrix_rows(s_in);
            }
            lds_barrier();
            if (cp >= 0) matrices(buf);
        }
    }
}

template <typename TI, int NMW, int KS, bool HB>
hipError_t launch_sweep(const BwdArgs &a, int32_t units, hipStream_t stream) {
    constexpr int NRB = 64 / (16 * NMW / KS);
    const size_t lds = (size_t)lay::TOTAL * sizeof(float);
    auto fn = dsweep_kernel<TI, NMW, KS, HB>;
    hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t blocks = NRB == 1 ? units : ((int64_t)units + 7) / 8 * 8 * NRB;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * (NMW + kPrepWaves)), lds, stream, a, units);
    return hipGetLastError();
}

template <typename TI, bool HB>
hipError_t launch_sweep_typed(const BwdArgs &a, hipStream_t stream) {
    const int S = a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B;
    const int32_t units = S * a.seg.H;
    const int nrb = row_blocks_for(units);
    if (nrb == 1) return launch_sweep<TI, 4, 1, HB>(a, units, stream);
    if (nrb == 2) return launch_sweep<TI, 4, 2, HB>(a, units, stream);
    return launch_sweep<TI, 2, 2, HB>(a, units, stream);
}

}  // namespace

hipError_t launch_backward_sweep(const BwdArgs &a, hipStream_t stream) {
    // bf16 streams with bf16 gradients: dS_C and drhs travel in bf16 (the
    // second pass's products round them to one bf16 piece anyway)
    if (a.dtype == 1) return a.grad_f32 ? launch_sweep_typed<uint16_t, false>(a, stream)
                                        : launch_sweep_typed<uint16_t, true>(a, stream);
    if (a.dtype == 2) return launch_sweep_typed<_Float16, false>(a, stream);
    return launch_sweep_typed<float, false>(a, stream);
}

}  // namespace wkv7
