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
// chunk is solved one phase later, while the state waves run its D1). With
// bf16 streams the products that feed only y run on bf16 MFMA with one piece
// per operand; with bf16 streams in 64-row workgroups every state product
// runs in split bf16 (three pieces) as well.
#include <type_traits>

#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr int kPrepWaves = 8;
constexpr int QLD = 68;    // row stride (floats) of 64-wide rows
constexpr int KLD = 36;    // row stride of the transposed [B^;K^] tile
constexpr int VLD = 20;    // row stride of the transposed V tile
constexpr int MLD = 20;    // row stride of the 16x16 matrices
// Split-path strides (words) are 2 mod 32, so that the 16 rows read by 16
// lanes with 8-byte loads cover 32 distinct banks.
constexpr int QAW = 34;    // words per bf16 row of 64 keys (split path)
constexpr int BKW = 50;    // words per key column of B^ and K^ pieces, 2 x 3 x 16 tokens
constexpr int VBW = 10;    // words per value row of V, 16 tokens
constexpr float kMinFactor = 9.313225746154785e-10f;  // 2^-30
constexpr float kFastMinW = 0.015625f;                 // 2^-6: fast chunks have every decay >= this

// Position of column c in a staged 64-float row: 4-column block b = c / 4
// sits at block 8 (b / 8) + (b + b / 8) % 8 (columns 0..31 in place, the upper
// half rotated by one block). With 32 four-byte LDS banks, the staging
// stores (eight lanes writing blocks 2k, then 2k + 1) and the column readers
// (32 lanes reading columns 0..31, then 32..63) each cover 32 distinct banks.
__device__ __forceinline__ int stage_block(int b) { return 8 * (b >> 3) + ((b + (b >> 3)) & 7); }
__device__ __forceinline__ int stage_pos(int c) { return 4 * stage_block(c >> 2) + (c & 3); }

enum { IR = 0, IW, IK, IA, IB, IV };
// acc += sum over 16 indices of a[e] v[e] (this lane's 4 of them), a fp32 in
// three bf16 pieces and v holding bf16 values: two K = 32 bf16 MFMAs
__device__ __forceinline__ f32x4 mm_k16_3v(f32x4 acc, float4 a, float4 v) {
    uint32_t h0, m0, l0, h1, m1, l1;
    split3(a.x, a.y, h0, m0, l0);
    split3(a.z, a.w, h1, m1, l1);
    const uint32_t v0 = pk_bf16(v.x, v.y), v1 = pk_bf16(v.z, v.w);
    acc = mfma_bf16_k32(u32x4_t{l0, l1, 0u, 0u}, u32x4_t{v0, v1, 0u, 0u}, acc);
    return mfma_bf16_k32(u32x4_t{h0, h1, m0, m1}, u32x4_t{v0, v1, v0, v1}, acc);
}
enum { MLAK = 0, MMRK, MMRB, MWI };

// LDS layout (floats): the operand waves' private rows, then two hand-off
// buffers (one per chunk parity) read by the state waves, then the key-split
// exchange. The hand-off buffer holds fp32 rows for the FP32-MFMA state path
// and bf16 pieces for the split-bf16 one.
template <bool SPLIT> struct Lay {
    // [2][6][16][64] r w k a b v, by chunk parity; column c of a row sits at
    // stage_pos(c)
    static constexpr int IN = 0;
    static constexpr int IN_SIZE = 6 * 16 * 64;
    static constexpr int AR = IN + 2 * IN_SIZE;        // [32][QLD] A'_t = a_t F_ex(t), R'_t = r_t F_in(t)
    static constexpr int AWR = AR + 32 * QLD;          // [8][QLD]  A'_t W_2, R'_t W_2 for t = 12..15
    static constexpr int BD = AWR + 8 * QLD;           // [16][QLD] b_s / F_s
    static constexpr int KD = BD + 16 * QLD;           // [16][QLD] k_s / F_s
    static constexpr int BL = KD + 16 * QLD;           // [32][QLD] b, k rows scaled to the split points
    static constexpr int LAB = BL + 32 * QLD;          // [16][MLD] L_ab (upper part stays zero)
    static constexpr int BUF = LAB + 16 * MLD;
    // within a hand-off buffer, FP32 path
    static constexpr int B_Q = 0;                      // [32][QLD] A^ (rows 0..15), R^ (16..31)
    static constexpr int B_BKT = B_Q + 32 * QLD;       // [64][KLD] B^ | K^ by key column j
    static constexpr int B_VT = B_BKT + 64 * KLD;      // [64][VLD] V by value row i
    // split-bf16 path (word offsets; a word holds two bf16)
    static constexpr int B_QA = 0;                     // [3 pieces][16 t][QAW] A^ by token, keys along the row
    static constexpr int B_QR = B_QA + 3 * 16 * QAW;   // [16 t][QAW] R^ (one piece)
    static constexpr int B_BK = B_QR + 16 * QAW;       // [64 j][BKW] B^ pieces, then K^ pieces, tokens along
    static constexpr int B_VB = B_BK + 64 * BKW;       // [64 i][VBW] V by value row, tokens along
    static constexpr int B_M = SPLIT ? B_VB + 64 * VBW : B_VT + 64 * VLD;   // [4][16][MLD] L_ak, M_rk, M_rb, W
    static constexpr int B_GC = B_M + 4 * 16 * MLD;    // [64] gamma_16
    static constexpr int BUF_SIZE = B_GC + 64;
    static constexpr int XCH = BUF + 2 * BUF_SIZE;     // [4 waves][2][64 lanes][4] partial D1 (key split)
    static constexpr int FLAGS = XCH + 4 * 2 * 256;    // [2 parities][2] fast-chunk flags (int)
    static constexpr int TOTAL = FLAGS + 4;
    // fast chunks of the split path: bf16 token rows (keys along the row) of
    // A- = A^ / gamma_16 (3 pieces), R- = R^ / gamma_16 (1), B^ (3), K^ (3),
    // in place of the split-point rows, which only other chunks use
    static constexpr int F_TA = AR;
    static constexpr int F_TR = F_TA + 3 * 16 * QAW;
    static constexpr int F_TB = F_TR + 16 * QAW;
    static constexpr int F_TK = F_TB + 3 * 16 * QAW;
    static_assert(F_TK + 3 * 16 * QAW <= LAB, "fast-path rows fit the split-point rows");
    static_assert(BUF % 4 == 0 && BUF_SIZE % 4 == 0 && B_M % 4 == 0 && B_GC % 4 == 0,
                  "16-byte aligned buffers");
};

template <typename TI, int NMW, int KS, bool SPLIT>
__global__ __launch_bounds__(64 * (NMW + kPrepWaves), 1) void fwd_ws_kernel(FwdArgs p, int32_t units) {
    using L = Lay<SPLIT>;
    static_assert(!SPLIT || sizeof(TI) == 2, "split path: 16-bit streams");
    // bf16 streams on the FP32-MFMA state path: the products that feed only
    // y (R^ S_0^T, M_rk V, M_rb X) round their operands to one bf16 piece and
    // run on bf16 MFMA, which leaves the SIMD's VALU to the operand waves; y
    // leaves in bf16 (2^-9). The state products against v (L_ak V, K^^T V)
    // take the fp32 operand in three bf16 pieces (24 bits) against v's
    // exact bf16 values; the others stay FP32
    constexpr bool kY1 = !SPLIT && std::is_same<TI, uint16_t>::value;
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
        float *xch_own = sm + L::XCH + wave * 512 + lane * 4;
        const float *xch_mate = sm + L::XCH + (rg + (1 - kh) * NG) * 512 + lane * 4;
        if constexpr (SPLIT) {
            // Split-bf16 products: every product that feeds the state takes
            // both operands in three bf16 pieces (six piece products, fp32
            // accumulation; see split3), the products that feed only y take
            // one piece each. bf16 MFMAs leave the VALU free for the other
            // waves on the SIMD, where FP32 MFMAs hold it.
            //
            // Contraction over keys (D1): element e of a lane's 8 covers key
            // 16 (q + e / 4) + 4 g + e % 4 of a tile pair (q, q + 1), which is
            // exactly the state's accumulator layout. Contraction over the 16
            // tokens of a chunk: elements 0-3 and 4-7 both cover tokens 4 g ..
            // 4 g + 3, each half carrying one piece, so one K = 32 MFMA takes
            // two piece products (a lone product leaves one half zero). Only
            // the K = 32 form is used: a K = 16 MFMA whose result feeds a
            // K = 32 one as its accumulator was measured to hand over stale
            // rows 4 g + 2, 4 g + 3 (no wait states were inserted between).
            constexpr int NP = NQ / 2;                   // key tile pairs per state wave
            const uint32_t *wbuf0 = (const uint32_t *)(sm + L::BUF);
#pragma unroll 1
            for (int c = 0; c <= nch; ++c) {
                const int cm = c - 1;
                const float *buf = sm + L::BUF + (cm & 1) * L::BUF_SIZE;
                const uint32_t *wbuf = wbuf0 + (cm & 1) * L::BUF_SIZE;
                f32x4 d1a = {0.f, 0.f, 0.f, 0.f}, d1r = d1a;
                u32x2_t vb = {0u, 0u};
                lds_barrier();
                // ---- phase X: checkpoint; D1 = [A^;R^] S_0^T; P_a += L_ak V
                if (cm >= 0) {
                    if (p.ckpt) {
                        float *cp = p.ckpt + ((u.ckpt + cm) * H + h) * (int64_t)(kN * kN) + (int64_t)irow * kN;
#pragma unroll
                        for (int qq = 0; qq < NQ; ++qq)
                            *(float4 *)(cp + 16 * (q0 + qq) + 4 * kq) =
                                make_float4(acc[qq][0], acc[qq][1], acc[qq][2], acc[qq][3]);
                    }
#pragma unroll
                    for (int P = 0; P < NP; ++P) {
                        const int q = q0 + 2 * P;
                        uint32_t hs[4], ms[4], ls[4];
                        split3(acc[2 * P][0], acc[2 * P][1], hs[0], ms[0], ls[0]);
                        split3(acc[2 * P][2], acc[2 * P][3], hs[1], ms[1], ls[1]);
                        split3(acc[2 * P + 1][0], acc[2 * P + 1][1], hs[2], ms[2], ls[2]);
                        split3(acc[2 * P + 1][2], acc[2 * P + 1][3], hs[3], ms[3], ls[3]);
                        const u32x4_t sh = {hs[0], hs[1], hs[2], hs[3]}, smd = {ms[0], ms[1], ms[2], ms[3]};
                        const u32x4_t sl = {ls[0], ls[1], ls[2], ls[3]};
                        auto rec = [&](int row) {            // keys of tiles q, q + 1 for this lane group
                            const uint32_t *r = wbuf + row * QAW + 8 * q + 2 * kq;
                            return cat(*(const u32x2_t *)r, *(const u32x2_t *)(r + 8));
                        };
                        const u32x4_t ah = rec(L::B_QA / QAW + l16), am = rec(L::B_QA / QAW + 16 + l16);
                        const u32x4_t al = rec(L::B_QA / QAW + 32 + l16), rh = rec(L::B_QR / QAW + l16);
                        d1a = mfma_bf16_k32(al, sh, d1a);
                        d1a = mfma_bf16_k32(ah, sl, d1a);
                        d1a = mfma_bf16_k32(am, smd, d1a);
                        d1r = mfma_bf16_k32(rh, sh, d1r);
                        d1a = mfma_bf16_k32(am, sh, d1a);
                        d1a = mfma_bf16_k32(ah, smd, d1a);
                        d1a = mfma_bf16_k32(ah, sh, d1a);
                    }
                    vb = *(const u32x2_t *)(wbuf + L::B_VB + irow * VBW + 2 * kq);
                    if (KS == 1 || kh == 0) {
                        const float4 lak = *(const float4 *)(buf + L::B_M + MLAK * 16 * MLD + l16 * MLD + 4 * kq);
                        uint32_t h0, m0, l0, h1, m1, l1;
                        split3(lak.x, lak.y, h0, m0, l0);
                        split3(lak.z, lak.w, h1, m1, l1);
                        d1a = mfma_bf16_k32(u32x4_t{l0, l1, 0u, 0u}, cat(vb, vb), d1a);
                        d1a = mfma_bf16_k32(u32x4_t{h0, h1, m0, m1}, cat(vb, vb), d1a);
                    }
                    if (KS > 1) {
                        *(float4 *)xch_own = make_float4(d1a[0], d1a[1], d1a[2], d1a[3]);
                        *(float4 *)(xch_own + 256) = make_float4(d1r[0], d1r[1], d1r[2], d1r[3]);
                    }
                }
                lds_barrier();
                // ---- phase Y: (add the partner's partial D1); X = W rhs;
                //      S^T = diag(gamma) S^T + K^^T V + B^^T X; Y = P_r + M_rb X
                //      + M_rk V; y out
                if (cm >= 0) {
                    if (KS > 1) {
                        const float4 pa = *(const float4 *)xch_mate;
                        const float4 pr = *(const float4 *)(xch_mate + 256);
                        d1a[0] += pa.x; d1a[1] += pa.y; d1a[2] += pa.z; d1a[3] += pa.w;
                        d1r[0] += pr.x; d1r[1] += pr.y; d1r[2] += pr.z; d1r[3] += pr.w;
                    }
                    const float4 wi = *(const float4 *)(buf + L::B_M + MWI * 16 * MLD + l16 * MLD + 4 * kq);
                    uint32_t rh0, rm0, rl0, rh1, rm1, rl1, wh0, wm0, wl0, wh1, wm1, wl1;
                    split3(d1a[0], d1a[1], rh0, rm0, rl0);
                    split3(d1a[2], d1a[3], rh1, rm1, rl1);
                    split3(wi.x, wi.y, wh0, wm0, wl0);
                    split3(wi.z, wi.w, wh1, wm1, wl1);
                    f32x4 xx = {0.f, 0.f, 0.f, 0.f};
                    xx = mfma_bf16_k32(u32x4_t{wl0, wl1, wh0, wh1}, u32x4_t{rh0, rh1, rl0, rl1}, xx);
                    xx = mfma_bf16_k32(u32x4_t{wh0, wh1, wm0, wm1}, u32x4_t{rm0, rm1, rm0, rm1}, xx);
                    xx = mfma_bf16_k32(u32x4_t{wh0, wh1, wm0, wm1}, u32x4_t{rh0, rh1, rh0, rh1}, xx);
                    uint32_t xh0, xm0, xl0, xh1, xm1, xl1;
                    split3(xx[0], xx[1], xh0, xm0, xl0);
                    split3(xx[2], xx[3], xh1, xm1, xl1);
#pragma unroll
                    for (int qq = 0; qq < NQ; ++qq) {
                        const int q = q0 + qq;
                        const float4 g4 = *(const float4 *)(buf + L::B_GC + 16 * q + 4 * kq);
                        const uint32_t *br = wbuf + L::B_BK + (16 * q + l16) * BKW + 2 * kq;
                        const u32x2_t bh = *(const u32x2_t *)br, bm = *(const u32x2_t *)(br + 8);
                        const u32x2_t bl = *(const u32x2_t *)(br + 16);
                        const u32x2_t kh_ = *(const u32x2_t *)(br + 24), km_ = *(const u32x2_t *)(br + 32);
                        const u32x2_t kl_ = *(const u32x2_t *)(br + 40);
                        f32x4 a = acc[qq];
                        a[0] *= g4.x; a[1] *= g4.y; a[2] *= g4.z; a[3] *= g4.w;
                        a = mfma_bf16_k32(u32x4_t{kl_.x, kl_.y, 0u, 0u}, cat(vb, vb), a);
                        a = mfma_bf16_k32(cat(kh_, km_), cat(vb, vb), a);
                        a = mfma_bf16_k32(cat(bl, bh), u32x4_t{xh0, xh1, xl0, xl1}, a);
                        a = mfma_bf16_k32(cat(bh, bm), u32x4_t{xm0, xm1, xm0, xm1}, a);
                        a = mfma_bf16_k32(cat(bh, bm), u32x4_t{xh0, xh1, xh0, xh1}, a);
                        acc[qq] = a;
                    }
                    if (KS == 1 || kh == 0) {
                        const float *mrow = buf + L::B_M + l16 * MLD + 4 * kq;
                        const float4 mrb = *(const float4 *)(mrow + MMRB * 16 * MLD);
                        const float4 mrk = *(const float4 *)(mrow + MMRK * 16 * MLD);
                        d1r = mfma_bf16_k32(u32x4_t{pk_bf16(mrb.x, mrb.y), pk_bf16(mrb.z, mrb.w),
                                                    pk_bf16(mrk.x, mrk.y), pk_bf16(mrk.z, mrk.w)},
                                            u32x4_t{xh0, xh1, vb.x, vb.y}, d1r);
                        const int t0 = cm * kChunk;
                        const int Lr = min(kChunk, u.len - t0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int t = 4 * kq + r;
                            if (t < Lr) IO<TI>::st((TI *)p.y, base + (int64_t)t0 * ts + row_off(t, ts, irow), d1r[r]);
                        }
                    }
                }
            }
        } else {
#pragma unroll 1
        for (int c = 0; c <= nch; ++c) {
            const int cm = c - 1;                        // chunk advanced in this iteration
            const float *buf = sm + L::BUF + (cm & 1) * L::BUF_SIZE;
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
                const float4 vb = *(const float4 *)(buf + L::B_VT + irow * VLD + 4 * kq);
                const float *mrow = buf + L::B_M + l16 * MLD + 4 * kq;
                const float4 lak = *(const float4 *)(mrow + MLAK * 16 * MLD);
                const float4 mrk = *(const float4 *)(mrow + MMRK * 16 * MLD);
                mrb = *(const float4 *)(mrow + MMRB * 16 * MLD);
                if constexpr (kY1) {
                    // state product on FP32 MFMA; the y-only R^ S_0^T as one
                    // bf16 MFMA per key tile pair (K = 32 keys)
#pragma unroll
                    for (int qq = 0; qq < NQ; ++qq) {
                        const float4 a4 = *(const float4 *)(buf + L::B_Q + l16 * QLD + 16 * (q0 + qq) + 4 * kq);
                        d1a = mfma4(a4.x, acc[qq][0], d1a);
                        d1a = mfma4(a4.y, acc[qq][1], d1a);
                        d1a = mfma4(a4.z, acc[qq][2], d1a);
                        d1a = mfma4(a4.w, acc[qq][3], d1a);
                    }
#pragma unroll
                    for (int qq = 0; qq < NQ; qq += 2) {
                        const float *rr = buf + L::B_Q + (16 + l16) * QLD + 16 * (q0 + qq) + 4 * kq;
                        const float4 r4 = *(const float4 *)rr, s4 = *(const float4 *)(rr + 16);
                        d1r = mfma_bf16_k32(
                            u32x4_t{pk_bf16(r4.x, r4.y), pk_bf16(r4.z, r4.w), pk_bf16(s4.x, s4.y), pk_bf16(s4.z, s4.w)},
                            u32x4_t{pk_bf16(acc[qq][0], acc[qq][1]), pk_bf16(acc[qq][2], acc[qq][3]),
                                    pk_bf16(acc[qq + 1][0], acc[qq + 1][1]), pk_bf16(acc[qq + 1][2], acc[qq + 1][3])},
                            d1r);
                    }
                } else {
#pragma unroll
                    for (int qq = 0; qq < NQ; ++qq) {
                        const int q = q0 + qq;
                        const float4 a4 = *(const float4 *)(buf + L::B_Q + l16 * QLD + 16 * q + 4 * kq);
                        const float4 r4 = *(const float4 *)(buf + L::B_Q + (16 + l16) * QLD + 16 * q + 4 * kq);
                        d1a = mfma4(a4.x, acc[qq][0], d1a);
                        d1r = mfma4(r4.x, acc[qq][0], d1r);
                        d1a = mfma4(a4.y, acc[qq][1], d1a);
                        d1r = mfma4(r4.y, acc[qq][1], d1r);
                        d1a = mfma4(a4.z, acc[qq][2], d1a);
                        d1r = mfma4(r4.z, acc[qq][2], d1r);
                        d1a = mfma4(a4.w, acc[qq][3], d1a);
                        d1r = mfma4(r4.w, acc[qq][3], d1r);
                    }
                }
                if (KS == 1 || kh == 0) {
                    if constexpr (kY1) {
                        d1a = mm_k16_3v(d1a, lak, vb);
                    } else {
                        d1a = mfma4(lak.x, vb.x, d1a); d1a = mfma4(lak.y, vb.y, d1a);
                        d1a = mfma4(lak.z, vb.z, d1a); d1a = mfma4(lak.w, vb.w, d1a);
                    }
                }
                if (KS == 1 || kh == 1) {
                    if constexpr (kY1) {
                        d1r = mfma_bf16_k32(u32x4_t{pk_bf16(mrk.x, mrk.y), pk_bf16(mrk.z, mrk.w), 0u, 0u},
                                            u32x4_t{pk_bf16(vb.x, vb.y), pk_bf16(vb.z, vb.w), 0u, 0u}, d1r);
                    } else {
                        d1r = mfma4(mrk.x, vb.x, d1r); d1r = mfma4(mrk.y, vb.y, d1r);
                        d1r = mfma4(mrk.z, vb.z, d1r); d1r = mfma4(mrk.w, vb.w, d1r);
                    }
                }
                if (KS > 1) {
                    *(float4 *)xch_own = make_float4(d1a[0], d1a[1], d1a[2], d1a[3]);
                    *(float4 *)(xch_own + 256) = make_float4(d1r[0], d1r[1], d1r[2], d1r[3]);
                }
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq) {
                    const int q = q0 + qq;
                    const float4 g4 = *(const float4 *)(buf + L::B_GC + 16 * q + 4 * kq);
                    const float *br = buf + L::B_BKT + (16 * q + l16) * KLD + 4 * kq;
                    bt[qq] = *(const float4 *)br;
                    const float4 k4 = *(const float4 *)(br + 16);
                    f32x4 a = acc[qq];
                    a[0] *= g4.x; a[1] *= g4.y; a[2] *= g4.z; a[3] *= g4.w;
                    if constexpr (kY1) {
                        a = mm_k16_3v(a, k4, vb);
                    } else {
                        a = mfma4(k4.x, vb.x, a); a = mfma4(k4.y, vb.y, a);
                        a = mfma4(k4.z, vb.z, a); a = mfma4(k4.w, vb.w, a);
                    }
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
                const float4 wi = *(const float4 *)(buf + L::B_M + MWI * 16 * MLD + l16 * MLD + 4 * kq);
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
                    if constexpr (kY1) {
                        d1r = mfma_bf16_k32(u32x4_t{pk_bf16(mrb.x, mrb.y), pk_bf16(mrb.z, mrb.w), 0u, 0u},
                                            u32x4_t{pk_bf16(xx[0], xx[1]), pk_bf16(xx[2], xx[3]), 0u, 0u}, d1r);
                    } else {
                        d1r = mfma4(mrb.x, xx[0], d1r); d1r = mfma4(mrb.y, xx[1], d1r);
                        d1r = mfma4(mrb.z, xx[2], d1r); d1r = mfma4(mrb.w, xx[3], d1r);
                    }
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
    float *s_AR = sm + L::AR;
    float *s_AWR = sm + L::AWR;
    float *s_BD = sm + L::BD;
    float *s_KD = sm + L::KD;
    float *s_BL = sm + L::BL;
    float *s_Lab = sm + L::LAB;

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
        float *s_in = sm + L::IN + (cc & 1) * L::IN_SIZE;
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
            if constexpr (SPLIT) {
                if (st == IW) {           // tokens 0-7 (operand wave 7) or 8-15 (wave 5)
                    bool ok = true;
#pragma unroll
                    for (int e = 0; e < 8; ++e) ok = ok && x[e] >= kFastMinW;
                    ok = __all(ok);
                    if (lane == 0) ((int *)(sm + L::FLAGS))[(cc & 1) * 2 + (pw == 7 ? 0 : 1)] = ok;
                }
            }
            // blocks e0 / 4 and e0 / 4 + 1 of the row (stage_pos)
            float *d = s_in + (st * 16 + t) * 64;
            *(float4 *)(d + 4 * stage_block(e0 >> 2)) = make_float4(x[0], x[1], x[2], x[3]);
            *(float4 *)(d + 4 * stage_block((e0 >> 2) + 1)) = make_float4(x[4], x[5], x[6], x[7]);
        }
    };

    // Per-column decay rows, lane = key column j. Each role reads all its inputs
    // before its first store (the stores go through runtime-offset pointers,
    // which would otherwise order every later load behind them).
    //
    // ---- phase X (operand waves 1-4): the rows the 16x16 matrices are built
    //      from: A' = a F_ex (wave 1), R' = r F_in (wave 2), b (3) and k (4) rows
    auto matrix_rows = [&](const float *s_in) {
        const int j = lane, pj = stage_pos(lane);
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
        const int j = lane, pj = stage_pos(lane);
        if constexpr (SPLIT) {
            if (pw == 7) {
                // B^ and K^ in three bf16 pieces each, by key column j with the
                // 16 tokens along (pieces of B^ at words 0, 8, 16, of K^ at 24,
                // 32, 40); V by value row j (bf16 streams: exact in one piece).
                // Eight tokens at a time, last ones first, to bound the live
                // registers beside the staging waves' loads in flight.
                float wv[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) wv[t] = s_in[IW * 1024 + t * 64 + pj];
                uint32_t *dst = (uint32_t *)(buf + L::B_BK) + j * BKW;
                uint32_t *vd = (uint32_t *)(buf + L::B_VB) + j * VBW;
                float d = 1.f;
#pragma unroll
                for (int hv = 1; hv >= 0; --hv) {
                    float xv[8], yv[8], vv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        xv[e] = s_in[IB * 1024 + (8 * hv + e) * 64 + pj];
                        yv[e] = s_in[IK * 1024 + (8 * hv + e) * 64 + pj];
                        vv[e] = s_in[IV * 1024 + (8 * hv + e) * 64 + pj];
                    }
#pragma unroll
                    for (int e = 7; e >= 0; --e) { xv[e] *= d; yv[e] *= d; d *= wv[8 * hv + e]; }
#pragma unroll
                    for (int sk = 0; sk < 2; ++sk) {
                        const float *x = sk ? yv : xv;
                        uint32_t ph[4], pm[4], pl[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) split3(x[2 * e], x[2 * e + 1], ph[e], pm[e], pl[e]);
                        uint32_t *o = dst + 24 * sk + 4 * hv;   // 8-byte aligned (BKW even)
                        *(uint2 *)o = make_uint2(ph[0], ph[1]);
                        *(uint2 *)(o + 2) = make_uint2(ph[2], ph[3]);
                        *(uint2 *)(o + 8) = make_uint2(pm[0], pm[1]);
                        *(uint2 *)(o + 10) = make_uint2(pm[2], pm[3]);
                        *(uint2 *)(o + 16) = make_uint2(pl[0], pl[1]);
                        *(uint2 *)(o + 18) = make_uint2(pl[2], pl[3]);
                    }
                    *(uint2 *)(vd + 4 * hv) = make_uint2(pk_bf16(vv[0], vv[1]), pk_bf16(vv[2], vv[3]));
                    *(uint2 *)(vd + 4 * hv + 2) = make_uint2(pk_bf16(vv[4], vv[5]), pk_bf16(vv[6], vv[7]));
                }
                return;
            }
        }
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
            if constexpr (SPLIT) {
                // A^ in three bf16 pieces and R^ in one, rows by token with the
                // 64 keys along the row (this lane writes key j of each row)
                uint16_t *qa = (uint16_t *)(buf + L::B_QA) + j, *qr = (uint16_t *)(buf + L::B_QR) + j;
#pragma unroll
                for (int t = 0; t < 16; t += 2) {
                    uint32_t hh, mm, ll;
                    split3(xv[t], xv[t + 1], hh, mm, ll);
                    const uint32_t rr = pk_bf16(yv[t], yv[t + 1]);
                    qa[t * 2 * QAW] = (uint16_t)hh;
                    qa[(t + 1) * 2 * QAW] = (uint16_t)(hh >> 16);
                    qa[(16 + t) * 2 * QAW] = (uint16_t)mm;
                    qa[(17 + t) * 2 * QAW] = (uint16_t)(mm >> 16);
                    qa[(32 + t) * 2 * QAW] = (uint16_t)ll;
                    qa[(33 + t) * 2 * QAW] = (uint16_t)(ll >> 16);
                    qr[t * 2 * QAW] = (uint16_t)rr;
                    qr[(t + 1) * 2 * QAW] = (uint16_t)(rr >> 16);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    buf[L::B_Q + t * QLD + j] = xv[t];
                    buf[L::B_Q + (16 + t) * QLD + j] = yv[t];
                }
            }
            buf[L::B_GC + j] = g;
        } else {
            float vv[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) vv[t] = s_in[IV * 1024 + t * 64 + pj];
            float d = 1.f;
#pragma unroll
            for (int s = 15; s >= 0; --s) { xv[s] *= d; yv[s] *= d; d *= wv[s]; }
            float *dst = buf + L::B_BKT + j * KLD;
#pragma unroll
            for (int s = 0; s < 16; s += 4) {
                *(float4 *)(dst + s) = make_float4(xv[s], xv[s + 1], xv[s + 2], xv[s + 3]);
                *(float4 *)(dst + 16 + s) = make_float4(yv[s], yv[s + 1], yv[s + 2], yv[s + 3]);
            }
#pragma unroll
            for (int t = 0; t < 16; t += 4)
                *(float4 *)(buf + L::B_VT + j * VLD + t) = make_float4(vv[t], vv[t + 1], vv[t + 2], vv[t + 3]);
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
                float *dst = isA ? (isB ? s_Lab : buf + L::B_M + MLAK * 16 * MLD)
                                 : buf + L::B_M + (isB ? MMRB : MMRK) * 16 * MLD;
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
            // quarter qtr covers columns 16 i + 4 qtr + e (the four quarters
            // of an item then read four distinct bank groups)
            const float *ar = s_AR + ((isL ? 0 : 16) + t) * QLD + 4 * qtr;
            const float *bd = s_BD + s * QLD + 4 * qtr;
            const float *kd = s_KD + s * QLD + 4 * qtr;
            float db = 0.f, dk = 0.f;
#pragma unroll
            for (int jj = 0; jj < 64; jj += 16) {
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
                float *mb = buf + L::B_M + t * MLD + s;
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

    // ==== fast chunks (split path, every decay >= 2^-6) ====
    // gamma_t >= 2^-96 stays far inside the fp32 range, so the pair decay
    // D_{t-1,s} = gamma_{t-1} / gamma_s is a product of the hand-off rows:
    // L_ab = A- B^^T, L_ak = A- K^^T, M_rb = R- B^^T, M_rk = R- K^^T with
    // A-_t = A^_t / gamma_16 = a_t gamma_{t-1} / gamma_16, R-_t = R^_t / gamma_16
    // and B^_s = b_s gamma_16 / gamma_s (each factor exact to rounding). The
    // split-point rows, their products and the within-sub-chunk VALU dot
    // products are not needed.
    auto fast_flag = [&](int cc) {
        const int *fl = (const int *)(sm + L::FLAGS) + (cc & 1) * 2;
        return fl[0] != 0 && fl[1] != 0;
    };
    // ---- phase X (operand waves 0-4): lane = key pair kp (keys 2 kp, 2 kp + 1)
    //      x token half th (tokens 8 th .. 8 th + 7), so that a word packs the
    //      two keys of one token. Role 1: A^ (3 pieces) by token, gamma_16;
    //      role 2: A- (3); roles 3, 4: B^, K^ (3 pieces each) by token for the
    //      tiles and by key column (token pairs) for the state waves; role 5
    //      (wave 0, after W of the previous chunk): R^, R- (1 piece each), V by
    //      value row.
    auto fast_rows = [&](const float *s_in, float *buf, int role) __attribute__((always_inline)) {
        const int kp = lane & 31, th = lane >> 5, t0 = 8 * th;
        const int pos = stage_pos(2 * kp);
        auto col2 = [&](int st, int t) { return *(const float2 *)(s_in + (st * 16 + t) * 64 + pos); };
        // decays of this lane's own tokens, and the products over the first
        // (g8) and the last (d8) eight tokens: each lane forms its own half's
        // product and takes the other half's from lane l ^ 32
        float2 wv[8], xv[8];
        float2 own = make_float2(1.f, 1.f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            wv[e] = col2(IW, t0 + e);
            own.x *= wv[e].x;
            own.y *= wv[e].y;
        }
        const float2 oth = make_float2(__shfl_xor(own.x, 32), __shfl_xor(own.y, 32));
        const float2 g8 = th ? oth : own, d8 = th ? own : oth;
        const int s1 = role <= 2 ? IA : role == 3 ? IB : role == 4 ? IK : IR;
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = col2(s1, t0 + e);
        uint32_t *wb = (uint32_t *)buf;
        if (role <= 2 || role == 5) {
            // A^_t = a_t gamma_{t-1} or R^_t = r_t gamma_t along this lane's
            // tokens, from gamma before its first token; A-, R- scale by
            // 1 / gamma_16
            const float2 g16 = make_float2(g8.x * d8.x, g8.y * d8.y);
            const float2 sc = make_float2(__builtin_amdgcn_rcpf(g16.x), __builtin_amdgcn_rcpf(g16.y));
            float2 g = th ? g8 : make_float2(1.f, 1.f);
            if (role <= 2) {
                uint32_t *qa = role == 1 ? wb + L::B_QA : (uint32_t *)(sm + L::F_TA);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = t0 + e;
                    float ax = xv[e].x * g.x, ay = xv[e].y * g.y;
                    if (role == 2) { ax *= sc.x; ay *= sc.y; }
                    g.x *= wv[e].x;
                    g.y *= wv[e].y;
                    uint32_t hh, mm, ll;
                    split3(ax, ay, hh, mm, ll);
                    qa[t * QAW + kp] = hh;
                    qa[(16 + t) * QAW + kp] = mm;
                    qa[(32 + t) * QAW + kp] = ll;
                }
                if (role == 1 && th == 1) *(float2 *)(buf + L::B_GC + 2 * kp) = g;    // gamma_16
            } else {
                uint32_t *qr = wb + L::B_QR, *tr = (uint32_t *)(sm + L::F_TR);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int t = t0 + e;
                    g.x *= wv[e].x;
                    g.y *= wv[e].y;
                    const float rx = xv[e].x * g.x, ry = xv[e].y * g.y;
                    qr[t * QAW + kp] = pk_bf16(rx, ry);
                    tr[t * QAW + kp] = pk_bf16(rx * sc.x, ry * sc.y);
                }
                // V by value row (rows 2 kp, 2 kp + 1), token pairs along
                float2 vv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) vv[e] = col2(IV, t0 + e);
                uint32_t *v0 = wb + L::B_VB + (2 * kp) * VBW + 4 * th, *v1 = v0 + VBW;
                *(uint2 *)v0 = make_uint2(pk_bf16(vv[0].x, vv[1].x), pk_bf16(vv[2].x, vv[3].x));
                *(uint2 *)(v0 + 2) = make_uint2(pk_bf16(vv[4].x, vv[5].x), pk_bf16(vv[6].x, vv[7].x));
                *(uint2 *)v1 = make_uint2(pk_bf16(vv[0].y, vv[1].y), pk_bf16(vv[2].y, vv[3].y));
                *(uint2 *)(v1 + 2) = make_uint2(pk_bf16(vv[4].y, vv[5].y), pk_bf16(vv[6].y, vv[7].y));
            }
        } else {
            // X^_s = x_s D_{16,s}, D built from the last token down
            float2 d = th ? make_float2(1.f, 1.f) : d8;
            uint32_t ph[8], pm[8], pl[8];
#pragma unroll
            for (int e = 7; e >= 0; --e) {
                split3(xv[e].x * d.x, xv[e].y * d.y, ph[e], pm[e], pl[e]);
                d.x *= wv[e].x;
                d.y *= wv[e].y;
            }
            uint32_t *tr = (uint32_t *)(sm + (role == 3 ? L::F_TB : L::F_TK));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                tr[(t0 + e) * QAW + kp] = ph[e];
                tr[(16 + t0 + e) * QAW + kp] = pm[e];
                tr[(32 + t0 + e) * QAW + kp] = pl[e];
            }
            // by key column: key 2 kp takes the low halves of two tokens' words,
            // key 2 kp + 1 the high halves
            uint32_t *k0 = wb + L::B_BK + (2 * kp) * BKW + 24 * (role - 3) + 4 * th, *k1 = k0 + BKW;
            auto by_key = [&](const uint32_t (&q)[8], int pc) {
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[e] = __builtin_amdgcn_perm(q[2 * e + 1], q[2 * e], 0x05040100u);
                    hi[e] = __builtin_amdgcn_perm(q[2 * e + 1], q[2 * e], 0x07060302u);
                }
                *(uint2 *)(k0 + 8 * pc) = make_uint2(lo[0], lo[1]);
                *(uint2 *)(k0 + 8 * pc + 2) = make_uint2(lo[2], lo[3]);
                *(uint2 *)(k1 + 8 * pc) = make_uint2(hi[0], hi[1]);
                *(uint2 *)(k1 + 8 * pc + 2) = make_uint2(hi[2], hi[3]);
            };
            by_key(ph, 0);
            by_key(pm, 1);
            by_key(pl, 2);
        }
    };

    // ---- phase Y (operand waves 0-2): the four 16x16 matrices on bf16 MFMA,
    //      K = 64 keys as two 32-key halves (element e of lane group g covers
    //      key 32 P + 8 g + e). Wave 0: L_ab (strictly lower, to the private
    //      L_ab), wave 1: L_ak, three pieces each; wave 2: M_rb and M_rk
    //      (lower with the diagonal), one piece each.
    auto fast_tiles = [&](float *buf) {
        const uint32_t *ta = (const uint32_t *)(sm + (pw == 2 ? L::F_TR : L::F_TA));
        auto rec = [&](const uint32_t *rows, int row, int P) {
            const uint32_t *r = rows + row * QAW + 16 * P + 4 * kq;
            return cat(*(const u32x2_t *)r, *(const u32x2_t *)(r + 2));
        };
        if (pw < 2) {
            const uint32_t *tb = (const uint32_t *)(sm + (pw == 0 ? L::F_TB : L::F_TK));
            f32x4 dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int P = 0; P < 2; ++P) {
                const u32x4_t ah = rec(ta, l16, P), am = rec(ta, 16 + l16, P), al = rec(ta, 32 + l16, P);
                const u32x4_t bh = rec(tb, l16, P), bm = rec(tb, 16 + l16, P), bl = rec(tb, 32 + l16, P);
                dd = mfma_bf16_k32(al, bh, dd);
                dd = mfma_bf16_k32(ah, bl, dd);
                dd = mfma_bf16_k32(am, bm, dd);
                dd = mfma_bf16_k32(am, bh, dd);
                dd = mfma_bf16_k32(ah, bm, dd);
                dd = mfma_bf16_k32(ah, bh, dd);
            }
            float *dst = pw == 0 ? s_Lab : buf + L::B_M + MLAK * 16 * MLD;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * kq + r;
                if (l16 < t) dst[t * MLD + l16] = dd[r];
            }
        } else {
            const uint32_t *tb = (const uint32_t *)(sm + L::F_TB), *tk = (const uint32_t *)(sm + L::F_TK);
            f32x4 mb = {0.f, 0.f, 0.f, 0.f}, mk = mb;
#pragma unroll
            for (int P = 0; P < 2; ++P) {
                const u32x4_t rr = rec(ta, l16, P);
                mb = mfma_bf16_k32(rr, rec(tb, l16, P), mb);
                mk = mfma_bf16_k32(rr, rec(tk, l16, P), mk);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * kq + r;
                if (l16 <= t) {
                    buf[L::B_M + MMRB * 16 * MLD + t * MLD + l16] = mb[r];
                    buf[L::B_M + MMRK * 16 * MLD + t * MLD + l16] = mk[r];
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
        for (int i = 0; i < 4; ++i) buf[L::B_M + MWI * 16 * MLD + (q + 4 * i) * MLD + col] = x[i];
    };

    // Entries of L_ab and of the hand-off matrices that are never written
    // (upper parts) stay zero.
    for (int q = ptid; q < 16 * MLD + 2 * L::BUF_SIZE; q += 64 * kPrepWaves) sm[L::LAB + q] = 0.f;
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
            float *buf = sm + L::BUF + (c & 1) * L::BUF_SIZE;
            const float *s_in = sm + L::IN + (c & 1) * L::IN_SIZE;
            lds_barrier();
            bool fast = false;
            if constexpr (SPLIT) {
                fast = c < nch && fast_flag(c);     // split path: staging in phase Y
            } else {
                if (c + 1 < nch) stage(c + 1, rw);
                issue(min(c + 1 + d, nch - 1), rw);
            }
            lds_barrier();
            if (c < nch && !fast) {
                if (pw == 5) matrices(buf);
                else handoff_rows(s_in, buf);
            }
            if constexpr (SPLIT) {
                if (c + 1 < nch) stage(c + 1, rw);
                issue(min(c + 1 + d, nch - 1), rw);
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
            float *buf = sm + L::BUF + (c & 1) * L::BUF_SIZE;
            const float *s_in = sm + L::IN + (c & 1) * L::IN_SIZE;
            lds_barrier();
            bool fast = false;
            if constexpr (SPLIT) fast = c < nch && fast_flag(c);
            if (pw == 0) {
                if (c >= 1) solve_w(sm + L::BUF + ((c - 1) & 1) * L::BUF_SIZE);
                if (fast) fast_rows(s_in, buf, 5);
            } else if (c < nch) {
                if (fast) fast_rows(s_in, buf, pw);
                else matrix_rows(s_in);
            }
            lds_barrier();
            if (c < nch) {
                if (!fast) matrices(buf);
                else if (pw < 3) fast_tiles(buf);
            }
        }
    }
}

template <typename TI, int NMW, int KS, bool SPLIT>
hipError_t launch_ws(const FwdArgs &a, int32_t units, hipStream_t stream) {
    constexpr int NRB = 64 / (16 * NMW / KS);
    const size_t lds = (size_t)Lay<SPLIT>::TOTAL * sizeof(float);
    auto fn = fwd_ws_kernel<TI, NMW, KS, SPLIT>;
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
    // bf16 streams in 64-row workgroups take the split-bf16 state path; the
    // narrower shapes repeat the operand work per row block, which the
    // split path makes heavier than it saves (measured: 32-row training
    // forward 0.49 ms FP32-MFMA against 0.51 ms split).
    constexpr bool SPLIT = std::is_same<TI, uint16_t>::value;
    const int nrb = row_blocks_for(units);
    if (nrb == 1) return launch_ws<TI, 4, 1, SPLIT>(a, units, stream);
    if (nrb == 2) return launch_ws<TI, 4, 2, false>(a, units, stream);
    return launch_ws<TI, 2, 2, false>(a, units, stream);
}

}  // namespace

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream) {
    if (a.dtype == 1) return launch_typed<uint16_t>(a, stream);
    if (a.dtype == 2) return launch_typed<_Float16>(a, stream);
    return launch_typed<float>(a, stream);
}

}  // namespace wkv7
