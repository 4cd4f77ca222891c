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
// (L_ak, M_rk the same with k_s).
//
// The 16x16 matrices. A pair decay splits at any token R with s < R <= t into
// two factors that are both <= 1: D_{t-1,s} = [prod_{R<=u<t} w_u] [prod_{s<u<R} w_u].
// With 4-token sub-chunks, every pair (t, s) in different sub-chunks has such a
// split point shared by a whole block: R = 8 for t in 8..15, s in 0..7; R = 4
// and R = 12 for the blocks (4..7, 0..3) and (12..15, 8..11). Those blocks are
// two 16x16x64 MFMA products of precomputed rows (a, r rows scaled from R; b, k
// rows scaled to R; the R = 4 and R = 12 blocks share one product whose two
// off-diagonal quadrants are discarded). Pairs inside one sub-chunk divide out
// the within-sub-chunk prefix F_s = prod_{4p<=u<=s} w_u instead, with every
// factor clamped to >= 2^-30 so F >= 2^-120 stays a normal fp32 number (w = 0
// then acts as 2^-30 on at most three neighbouring tokens); they are VALU dot
// products. W = (I - L_ab)^-1 comes from column-wise forward substitution.
//
// Work split (warp specialisation): a workgroup owns RB = 16*NMW/KS value
// rows of one (sequence, head) and has NMW "state" waves and 8 "operand"
// waves. Only the state waves touch the state: each holds 16 rows x 64/KS
// columns of S in MFMA accumulators as S^T tiles (lane l holds S[row0 +
// l%16][16*jt + 4*(l/16) + r]), which is directly the B operand of the next
// chunk's [A^;R^] S_0^T product, and the D1 -> chain -> D2 sequence of a chunk
// stays in registers (the chain's outputs come out in the B-operand layout of
// the next product). With KS = 2 the two waves that share 16 rows each hold
// half of the key columns, so the serial per-chunk MFMA chain is spread over
// all four SIMDs when a workgroup has only 32 rows; their partial D1 sums
// (over their key columns) meet in LDS. The operand waves stage inputs and build everything that does
// not depend on the state (decay rows, the 16x16 matrices, W) for chunk c
// while the state waves advance through chunk c-1; the two sides meet through
// a double-buffered LDS hand-off, two workgroup barriers per chunk (W of a
// chunk is solved one phase later, while the state waves run its D1).
#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr int kPrepWaves = 8;
constexpr int QLD = 68;    // row stride (floats) of 64-wide rows
constexpr int KLD = 36;    // row stride of the transposed [B^;K^] tile
constexpr int VLD = 20;    // row stride of the transposed V tile
constexpr int MLD = 20;    // row stride of the 16x16 matrices
constexpr float kMinFactor = 9.313225746154785e-10f;  // 2^-30

enum { IR = 0, IW, IK, IA, IB, IV };
enum { MLAK = 0, MMRK, MMRB, MWI };

// LDS layout (floats): the operand waves' private rows, then two hand-off
// buffers (one per chunk parity) read by the state waves.
namespace lay {
// [2][6][16][64] r w k a b v, by chunk parity; column c of a row sits at
// 32 (c & 4 ? 1 : 0) + 4 (c >> 3) + (c & 3)
constexpr int IN = 0;
constexpr int IN_SIZE = 6 * 16 * 64;
constexpr int AR = IN + 2 * IN_SIZE;        // [32][QLD] A'_t = a_t F_ex(t), R'_t = r_t F_in(t)
constexpr int AWR = AR + 32 * QLD;          // [8][QLD]  A'_t W_2, R'_t W_2 for t = 12..15
constexpr int BD = AWR + 8 * QLD;           // [16][QLD] b_s / F_s
constexpr int KD = BD + 16 * QLD;           // [16][QLD] k_s / F_s
constexpr int BL = KD + 16 * QLD;           // [32][QLD] b, k rows scaled to the split points
constexpr int LAB = BL + 32 * QLD;          // [16][MLD] L_ab (upper part stays zero)
constexpr int BUF = LAB + 16 * MLD;
// within a hand-off buffer
constexpr int B_Q = 0;                      // [32][QLD] A^ (rows 0..15), R^ (16..31)
constexpr int B_BKT = B_Q + 32 * QLD;       // [64][KLD] B^ | K^ by key column j
constexpr int B_VT = B_BKT + 64 * KLD;      // [64][VLD] V by value row i
constexpr int B_M = B_VT + 64 * VLD;        // [4][16][MLD] L_ak, M_rk, M_rb, W
constexpr int B_GC = B_M + 4 * 16 * MLD;    // [64] gamma_16
constexpr int BUF_SIZE = B_GC + 64;
constexpr int XCH = BUF + 2 * BUF_SIZE;     // [4 waves][2][64 lanes][4] partial D1 (key split)
constexpr int TOTAL = XCH + 4 * 2 * 256;
static_assert(BUF % 4 == 0 && BUF_SIZE % 4 == 0, "16-byte aligned buffers");
}  // namespace lay

template <typename TI, int NMW, int KS>
__global__ __launch_bounds__(64 * (NMW + kPrepWaves), 1) void fwd_ws_kernel(FwdArgs p, int32_t units) {
    constexpr int NG = NMW / KS;       // 16-row groups per workgroup
    constexpr int RB = 16 * NG;        // value rows per workgroup
    constexpr int NRB = 64 / RB;       // row blocks per unit
    constexpr int NQ = 4 / KS;         // 16-column key tiles per state wave
    static_assert(KS == 1 || KS == 2, "key split of 1 or 2");
    extern __shared__ __align__(16) float sm[];

    // Workgroup -> (unit, row block). Row blocks of one unit go to the same
    // XCD (workgroups are dealt to the 8 XCDs round robin) so that their
    // shared reads of the inputs hit one L2.
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
        f32x4 acc[NQ];
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
            if (p.s0) {
                const float4 v4 = *(const float4 *)(p.s0 + sbase + (int64_t)irow * kN + 16 * (q0 + qq) + 4 * kq);
                acc[qq] = f32x4{v4.x, v4.y, v4.z, v4.w};
            } else {
                acc[qq] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        float *xch_own = sm + lay::XCH + wave * 512 + lane * 4;
        const float *xch_mate = sm + lay::XCH + (rg + (1 - kh) * NG) * 512 + lane * 4;
#pragma unroll 1
        for (int c = 0; c <= nch; ++c) {
            const int cm = c - 1;                        // chunk advanced in this iteration
            const float *buf = sm + lay::BUF + (cm & 1) * lay::BUF_SIZE;
            f32x4 d1a = {0.f, 0.f, 0.f, 0.f}, d1r = d1a;
            float4 bt[NQ];                               // B^ rows of this wave's state tiles
            float4 mrb = make_float4(0.f, 0.f, 0.f, 0.f);
            lds_barrier();
            // ---- phase X (W of this chunk is being solved meanwhile):
            //      checkpoint; D1 = [A^;R^] S_0^T for this wave's rows (over its
            //      key columns); P_a += L_ak V, P_r += M_rk V (one of them per
            //      key part when split); S^T = diag(gamma) S^T + K^^T V
            if (cm >= 0) {
                if (p.ckpt) {
                    float *cp = p.ckpt + ((u.ckpt + cm) * H + h) * (int64_t)(kN * kN) + (int64_t)irow * kN;
#pragma unroll
                    for (int qq = 0; qq < NQ; ++qq)
                        *(float4 *)(cp + 16 * (q0 + qq) + 4 * kq) =
                            make_float4(acc[qq][0], acc[qq][1], acc[qq][2], acc[qq][3]);
                }
                const float4 vb = *(const float4 *)(buf + lay::B_VT + irow * VLD + 4 * kq);
                const float *mrow = buf + lay::B_M + l16 * MLD + 4 * kq;
                const float4 lak = *(const float4 *)(mrow + MLAK * 16 * MLD);
                const float4 mrk = *(const float4 *)(mrow + MMRK * 16 * MLD);
                mrb = *(const float4 *)(mrow + MMRB * 16 * MLD);
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq) {
                    const int q = q0 + qq;
                    const float4 a4 = *(const float4 *)(buf + lay::B_Q + l16 * QLD + 16 * q + 4 * kq);
                    const float4 r4 = *(const float4 *)(buf + lay::B_Q + (16 + l16) * QLD + 16 * q + 4 * kq);
                    d1a = mfma4(a4.x, acc[qq][0], d1a);
                    d1r = mfma4(r4.x, acc[qq][0], d1r);
                    d1a = mfma4(a4.y, acc[qq][1], d1a);
                    d1r = mfma4(r4.y, acc[qq][1], d1r);
                    d1a = mfma4(a4.z, acc[qq][2], d1a);
                    d1r = mfma4(r4.z, acc[qq][2], d1r);
                    d1a = mfma4(a4.w, acc[qq][3], d1a);
                    d1r = mfma4(r4.w, acc[qq][3], d1r);
                }
                if (KS == 1 || kh == 0) {
                    d1a = mfma4(lak.x, vb.x, d1a); d1a = mfma4(lak.y, vb.y, d1a);
                    d1a = mfma4(lak.z, vb.z, d1a); d1a = mfma4(lak.w, vb.w, d1a);
                }
                if (KS == 1 || kh == 1) {
                    d1r = mfma4(mrk.x, vb.x, d1r); d1r = mfma4(mrk.y, vb.y, d1r);
                    d1r = mfma4(mrk.z, vb.z, d1r); d1r = mfma4(mrk.w, vb.w, d1r);
                }
                if (KS > 1) {
                    *(float4 *)xch_own = make_float4(d1a[0], d1a[1], d1a[2], d1a[3]);
                    *(float4 *)(xch_own + 256) = make_float4(d1r[0], d1r[1], d1r[2], d1r[3]);
                }
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq) {
                    const int q = q0 + qq;
                    const float4 g4 = *(const float4 *)(buf + lay::B_GC + 16 * q + 4 * kq);
                    const float *br = buf + lay::B_BKT + (16 * q + l16) * KLD + 4 * kq;
                    bt[qq] = *(const float4 *)br;
                    const float4 k4 = *(const float4 *)(br + 16);
                    f32x4 a = acc[qq];
                    a[0] *= g4.x; a[1] *= g4.y; a[2] *= g4.z; a[3] *= g4.w;
                    a = mfma4(k4.x, vb.x, a); a = mfma4(k4.y, vb.y, a);
                    a = mfma4(k4.z, vb.z, a); a = mfma4(k4.w, vb.w, a);
                    acc[qq] = a;
                }
            }
            lds_barrier();
            // ---- phase Y: (add the partner's partial D1); X = W rhs;
            //      Y = P_r + M_rk V + M_rb X; y out; S^T += B^^T X
            if (cm >= 0) {
                if (KS > 1) {
                    const float4 pa = *(const float4 *)xch_mate;
                    const float4 pr = *(const float4 *)(xch_mate + 256);
                    d1a[0] += pa.x; d1a[1] += pa.y; d1a[2] += pa.z; d1a[3] += pa.w;
                    d1r[0] += pr.x; d1r[1] += pr.y; d1r[2] += pr.z; d1r[3] += pr.w;
                }
                const float4 wi = *(const float4 *)(buf + lay::B_M + MWI * 16 * MLD + l16 * MLD + 4 * kq);
                f32x4 xx = {0.f, 0.f, 0.f, 0.f};
                xx = mfma4(wi.x, d1a[0], xx); xx = mfma4(wi.y, d1a[1], xx);
                xx = mfma4(wi.z, d1a[2], xx); xx = mfma4(wi.w, d1a[3], xx);
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq) {
                    f32x4 a = acc[qq];
                    a = mfma4(bt[qq].x, xx[0], a); a = mfma4(bt[qq].y, xx[1], a);
                    a = mfma4(bt[qq].z, xx[2], a); a = mfma4(bt[qq].w, xx[3], a);
                    acc[qq] = a;
                }
                if (KS == 1 || kh == 0) {
                    d1r = mfma4(mrb.x, xx[0], d1r); d1r = mfma4(mrb.y, xx[1], d1r);
                    d1r = mfma4(mrb.z, xx[2], d1r); d1r = mfma4(mrb.w, xx[3], d1r);
                    const int t0 = cm * kChunk;
                    const int L = min(kChunk, u.len - t0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 4 * kq + r;
                        if (t < L) IO<TI>::st((TI *)p.y, base + (int64_t)t0 * ts + row_off(t, ts, irow), d1r[r]);
                    }
                }
            }
        }
        if (p.s_out) {
            float *op = p.s_out + sbase + (int64_t)irow * kN;
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq)
                *(float4 *)(op + 16 * (q0 + qq) + 4 * kq) = make_float4(acc[qq][0], acc[qq][1], acc[qq][2], acc[qq][3]);
        }
        return;
    }

    // ================= operand waves =================
    const int pw = wave - NMW;                 // 0..7, uniform
    const int ptid = tid - 64 * NMW;           // 0..511
    const int sid = ptid - 320;                // staging thread index (operand waves 5..7)
    float *s_AR = sm + lay::AR;
    float *s_AWR = sm + lay::AWR;
    float *s_BD = sm + lay::BD;
    float *s_KD = sm + lay::KD;
    float *s_BL = sm + lay::BL;
    float *s_Lab = sm + lay::LAB;

    // Staging (operand waves 5-7): element group g = sid + 192k (k = 0..3) of
    // 6 streams x 16 tokens x 8 groups of 8 elements; stream g >> 7 is uniform
    // per wave. Loads are issued unconditionally (chunk index and token rows
    // clamped into the sequence), so that the registers in flight have exactly
    // one definition per iteration. For 16-bit inputs two register sets
    // alternate, which keeps each chunk's loads in flight for two chunk
    // periods (HBM latency under load exceeds one); fp32 inputs have room for
    // one set only.
    constexpr bool kTwoSets = sizeof(TI) == 2;
    Raw<TI, 4> raw, raw1;
    const TI *sp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int st = __builtin_amdgcn_readfirstlane((sid + 192 * k) >> 7);
        const void *vp = st == IR ? p.r : st == IW ? p.w : st == IK ? p.k
                       : st == IA ? p.a : st == IB ? p.b : p.v;
        sp[k] = (const TI *)vp + base;
    }
    auto issue = [&](int cc, Raw<TI, 4> &raw) {      // 0 <= cc < nch
        const int Lc = min(kChunk, u.len - cc * kChunk);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int g = sid + 192 * k;
            const int t = min((g >> 3) & 15, Lc - 1), e0 = (g & 7) * 8;
            raw_load(sp[k] + (int64_t)(cc * kChunk) * ts + row_off(t, ts, e0), raw, k);
        }
    };
    auto stage = [&](int cc, const Raw<TI, 4> &raw) {
        const int Lc = min(kChunk, u.len - cc * kChunk);
        float *s_in = sm + lay::IN + (cc & 1) * lay::IN_SIZE;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int g = sid + 192 * k;
            const int st = g >> 7, t = (g >> 3) & 15, e0 = (g & 7) * 8;
            // unpacked unconditionally, then replaced by identity tokens past
            // the end (a branch would leave the loads pending on one path)
            float x[8];
            raw_unpack(raw, k, x);
            if (st == IW) decay_of<8>(x, p.logw);
            const float f = st == IW ? 1.f : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = t < Lc ? x[e] : f;
            // columns e0..e0+3 to 4 (g & 7) and e0+4..e0+7 to 32 + 4 (g & 7):
            // each store instruction covers whole 128-byte row segments
            float *d = s_in + (st * 16 + t) * 64 + (e0 >> 1);
            *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
            *(float4 *)(d + 32) = make_float4(x[4], x[5], x[6], x[7]);
        }
    };

    // Per-column decay rows, lane = key column j. Each role reads all its inputs
    // before its first store (the stores go through runtime-offset pointers,
    // which would otherwise order every later load behind them).
    //
    // ---- phase X (operand waves 1-4): the rows the 16x16 matrices are built
    //      from: A' = a F_ex (wave 1), R' = r F_in (wave 2), b (3) and k (4) rows
    auto matrix_rows = [&](const float *s_in) {
        const int j = lane, pj = ((lane & 4) << 3) + ((lane >> 3) << 2) + (lane & 3);
        const int role = pw - 1;
        const int st = role == 0 ? IA : role == 1 ? IR : role == 2 ? IB : IK;
        float wv[16], xv[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            wv[t] = s_in[IW * 1024 + t * 64 + pj];
            xv[t] = s_in[st * 1024 + t * 64 + pj];
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
                    const float wc = fmaxf(wv[t], kMinFactor);
                    if (inc) f *= wc;
                    o[t] = xv[t] * f;
                    if (!inc) f *= wc;
                }
            }
            const float W2 = (wv[8] * wv[9]) * (wv[10] * wv[11]);
#pragma unroll
            for (int t = 0; t < 16; ++t) s_AR[(16 * inc + t) * QLD + j] = o[t];
#pragma unroll
            for (int e = 0; e < 4; ++e) s_AWR[(4 * inc + e) * QLD + j] = o[12 + e] * W2;
        } else {                   // x_s / F_s, and x_s scaled to the split points
            const int ko = role - 2;           // row offset of the k rows in BL
            float od[16], os[12];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float suf = 1.f;                 // suf = prod_{s<u<4q+4} w_u, built downwards
#pragma unroll
                for (int e = 3; e >= 0; --e) {
                    if (q < 3) os[4 * q + e] = xv[4 * q + e] * suf;
                    suf *= wv[4 * q + e];
                }
                // 1 / F_s (factors clamped) from one reciprocal of the
                // sub-chunk's product F_{4q+3}, then 1 / F_{s-1} = w_s / F_s
                float wc[4], F = 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wc[e] = fmaxf(wv[4 * q + e], kMinFactor);
                    F *= wc[e];
                }
                float inv = __builtin_amdgcn_rcpf(F);
#pragma unroll
                for (int e = 3; e >= 0; --e) {
                    od[4 * q + e] = xv[4 * q + e] * inv;
                    inv *= wc[e];
                }
            }
            const float W1 = (wv[4] * wv[5]) * (wv[6] * wv[7]);
            float *dd = ko ? s_KD : s_BD;
#pragma unroll
            for (int s = 0; s < 16; ++s) dd[s * QLD + j] = od[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s_BL[(8 * ko + e) * QLD + j] = os[e] * W1;          // s = e scaled to 8
                s_BL[(16 + 4 * ko + e) * QLD + j] = os[e];          // s = e scaled to 4
                s_BL[(8 * ko + 4 + e) * QLD + j] = os[4 + e];       // s = 4+e scaled to 8
                s_BL[(24 + 4 * ko + e) * QLD + j] = os[8 + e];      // s = 8+e scaled to 12
            }
        }
    };

    // ---- phase Y (operand waves 6, 7): the hand-off rows for the state waves:
    //      A^_t = a_t gamma_{t-1}, R^_t = r_t gamma_t, gamma_16 (wave 6);
    //      B^, K^ by key column and V by value row (wave 7)
    auto handoff_rows = [&](const float *s_in, float *buf) {
        const int j = lane, pj = ((lane & 4) << 3) + ((lane >> 3) << 2) + (lane & 3);
        float wv[16], xv[16], yv[16];
        const int s1 = pw == 6 ? IA : IB, s2 = pw == 6 ? IR : IK;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            wv[t] = s_in[IW * 1024 + t * 64 + pj];
            xv[t] = s_in[s1 * 1024 + t * 64 + pj];
            yv[t] = s_in[s2 * 1024 + t * 64 + pj];
        }
        if (pw == 6) {
            float g = 1.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                xv[t] *= g;
                g *= wv[t];
                yv[t] *= g;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                buf[lay::B_Q + t * QLD + j] = xv[t];
                buf[lay::B_Q + (16 + t) * QLD + j] = yv[t];
            }
            buf[lay::B_GC + j] = g;
        } else {
            float vv[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) vv[t] = s_in[IV * 1024 + t * 64 + pj];
            float d = 1.f;
#pragma unroll
            for (int s = 15; s >= 0; --s) { xv[s] *= d; yv[s] *= d; d *= wv[s]; }
            float *dst = buf + lay::B_BKT + j * KLD;
#pragma unroll
            for (int s = 0; s < 16; s += 4) {
                *(float4 *)(dst + s) = make_float4(xv[s], xv[s + 1], xv[s + 2], xv[s + 3]);
                *(float4 *)(dst + 16 + s) = make_float4(yv[s], yv[s + 1], yv[s + 2], yv[s + 3]);
            }
#pragma unroll
            for (int t = 0; t < 16; t += 4)
                *(float4 *)(buf + lay::B_VT + j * VLD + t) = make_float4(vv[t], vv[t + 1], vv[t + 2], vv[t + 3]);
        }
    };

    // ---- phase Y (operand waves 0-5): the 16x16 matrices. Waves 0, 1: the
    //      cross-sub-chunk blocks on MFMA; waves 2-5: the within-sub-chunk pairs on VALU
    auto matrices = [&](float *buf) {
        if (pw < 2) {
            // wave 0: split at 8: rows m < 8 are a rows t = 8+m, m >= 8 r rows t = m;
            //         columns n < 8 are b rows s = n, n >= 8 k rows s = n-8.
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
                    isB = n < 8;  s = isB ? n : n - 8;
                } else {
                    isA = (mm & 4) == 0; t = isA ? 4 + mm : mm;
                    isB = (n & 4) == 0;  s = isB ? n : n - 4;
                    valid = (mm < 8) == (n < 8);
                }
                float *dst = isA ? (isB ? s_Lab : buf + lay::B_M + MLAK * 16 * MLD)
                                 : buf + lay::B_M + (isB ? MMRB : MMRK) * 16 * MLD;
                if (valid) dst[t * MLD + s] = d[r];
            }
        } else if (pw < 6) {
            // 64 items (sub-chunk p, pair k) x 4 quarters of the 64 columns
            const int dt = ptid - 128;
            const int item = dt >> 2, qtr = dt & 3;
            const int sc = item >> 4, k = item & 15;
            int et, es;
            const bool isL = k < 6;
            if (isL) {                 // s < t
                et = 1 + (k >= 1) + (k >= 3);
                es = k - et * (et - 1) / 2;
            } else {                   // s <= t
                const int mi = k - 6;
                et = (mi >= 1) + (mi >= 3) + (mi >= 6);
                es = mi - et * (et + 1) / 2;
            }
            const int t = 4 * sc + et, s = 4 * sc + es;
            const float *ar = s_AR + ((isL ? 0 : 16) + t) * QLD + 16 * qtr;
            const float *bd = s_BD + s * QLD + 16 * qtr;
            const float *kd = s_KD + s * QLD + 16 * qtr;
            float db = 0.f, dk = 0.f;
#pragma unroll
            for (int jj = 0; jj < 16; jj += 4) {
                const float4 x = *(const float4 *)(ar + jj);
                const float4 b = *(const float4 *)(bd + jj);
                const float4 kk = *(const float4 *)(kd + jj);
                db = fmaf(x.x, b.x, db); dk = fmaf(x.x, kk.x, dk);
                db = fmaf(x.y, b.y, db); dk = fmaf(x.y, kk.y, dk);
                db = fmaf(x.z, b.z, db); dk = fmaf(x.z, kk.z, dk);
                db = fmaf(x.w, b.w, db); dk = fmaf(x.w, kk.w, dk);
            }
            db = quad_sum(db);
            dk = quad_sum(dk);
            if (qtr == 0) {
                float *mb = buf + lay::B_M + t * MLD + s;
                if (isL) {
                    s_Lab[t * MLD + s] = db;
                    mb[MLAK * 16 * MLD] = dk;
                } else {
                    mb[MMRB * 16 * MLD] = db;
                    mb[MMRK * 16 * MLD] = dk;
                }
            }
        }
    };

    // ---- W = (I - L_ab)^-1 (one wave: column c = lane / 4, rows t = lane % 4 + 4i
    //      held by the 4 lanes of a quad, forward substitution over s)
    auto solve_w = [&](float *buf) {
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
#pragma unroll
        for (int i = 0; i < 4; ++i) buf[lay::B_M + MWI * 16 * MLD + (q + 4 * i) * MLD + col] = x[i];
    };

    // Entries of L_ab and of the hand-off matrices that are never written
    // (upper parts) stay zero.
    for (int q = ptid; q < 16 * MLD + 2 * lay::BUF_SIZE; q += 64 * kPrepWaves) sm[lay::LAB + q] = 0.f;
    if (nch == 0) {            // nothing to build; match the state waves' two barriers
        lds_barrier();
        lds_barrier();
        return;
    }

    // Per iteration c: phase X builds the matrix rows of chunk c, solves W of
    // chunk c-1 and stages chunk c+1; phase Y builds the 16x16 matrices and the
    // hand-off rows of chunk c. The state waves advance chunk c-1 meanwhile and
    // need W only in phase Y.
    if (pw >= 5) {
        // iteration c stages chunk c+1 from set rw and refills rw with chunk
        // c+1+d (d = 2 with two sets, else 1)
        auto step = [&](int c, Raw<TI, 4> &rw, int d) {
            float *buf = sm + lay::BUF + (c & 1) * lay::BUF_SIZE;
            const float *s_in = sm + lay::IN + (c & 1) * lay::IN_SIZE;
            lds_barrier();
            if (c + 1 < nch) stage(c + 1, rw);
            issue(min(c + 1 + d, nch - 1), rw);
            lds_barrier();
            if (c < nch) {
                if (pw == 5) matrices(buf);
                else handoff_rows(s_in, buf);
            }
        };
        issue(0, raw);
        stage(0, raw);
        if constexpr (kTwoSets) {
            issue(min(1, nch - 1), raw1);
            // keep every load of chunk 1 ahead of chunk 2's, so that staging
            // chunk 1 waits for its own loads only
            __builtin_amdgcn_sched_barrier(0);
            issue(min(2, nch - 1), raw);
#pragma unroll 1
            for (int c = 0; c <= nch; c += 2) {
                step(c, raw1, 2);                  // chunk c+1 was loaded into raw1
                if (c + 1 > nch) break;
                step(c + 1, raw, 2);               // chunk c+2 was loaded into raw
            }
        } else {
            issue(min(1, nch - 1), raw);
#pragma unroll 1
            for (int c = 0; c <= nch; ++c) step(c, raw, 1);
        }
    } else {
#pragma unroll 1
        for (int c = 0; c <= nch; ++c) {
            float *buf = sm + lay::BUF + (c & 1) * lay::BUF_SIZE;
            const float *s_in = sm + lay::IN + (c & 1) * lay::IN_SIZE;
            lds_barrier();
            if (pw == 0) {
                if (c >= 1) solve_w(sm + lay::BUF + ((c - 1) & 1) * lay::BUF_SIZE);
            } else if (c < nch) {
                matrix_rows(s_in);
            }
            lds_barrier();
            if (c < nch) matrices(buf);
        }
    }
}

template <typename TI, int NMW, int KS>
hipError_t launch_ws(const FwdArgs &a, int32_t units, hipStream_t stream) {
    constexpr int NRB = 64 / (16 * NMW / KS);
    const size_t lds = (size_t)lay::TOTAL * sizeof(float);
    auto fn = fwd_ws_kernel<TI, NMW, KS>;
    hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t blocks = NRB == 1 ? units : ((int64_t)units + 7) / 8 * 8 * NRB;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * (NMW + kPrepWaves)), lds, stream, a, units);
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_typed(const FwdArgs &a, hipStream_t stream) {
    const int S = a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B;
    const int32_t units = S * a.seg.H;
    // One workgroup per CU (LDS); split value rows across workgroups when
    // there are fewer units than CUs, and then key columns across the state
    // waves that share rows.
    if (units >= 256) return launch_ws<TI, 4, 1>(a, units, stream);
    if (units >= 128) return launch_ws<TI, 4, 2>(a, units, stream);
    return launch_ws<TI, 2, 2>(a, units, stream);
}

}  // namespace

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream) {
    if (a.dtype == 1) return launch_typed<uint16_t>(a, stream);
    if (a.dtype == 2) return launch_typed<_Float16>(a, stream);
    return launch_typed<float>(a, stream);
}

}  // namespace wkv7
