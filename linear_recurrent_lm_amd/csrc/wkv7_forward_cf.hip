// WKV-7 forward in chunk form (C = 16) on MFMA, one lean workgroup per
// (sequence, head): N / 16 waves, wave w holding value rows 16 w .. 16 w + 15
// of the state in MFMA accumulators. Dense batches, or one workgroup per
// (sequence of a segment table, head).
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
// factor to rounding): four MFMA products (with bf16 streams the 1 / gamma_15
// goes on the B^ and K^ side instead). Other chunks form the entries as dot
// products with the decay products taken pair by pair (VALU). W =
// (I - L_ab)^-1 comes from forward substitution by one wave.
//
// Two arithmetic layouts. fp32 and fp16 streams take every product on FP32
// MFMA (16x16x4). bf16 streams take them on bf16 MFMA (16x16x32) in split
// form: each operand of a product that feeds the state is carried as three
// bf16 pieces (x = h + m + l, 24 significant bits) and six piece products
// accumulate in fp32, which reproduces the fp32 product; V needs one piece
// (its values are bf16), and the products that feed only y take fewer. On
// gfx950 FP32 MFMAs hold the SIMD's VALU while they run and bf16 MFMAs do
// not, so the split form also lets the row and staging work overlap them.
//
// Per chunk, three LDS barriers (four on chunks with small decays): the
// prefix and suffix products and the scaled rows (one thread per key and row
// kind); the dense products A^ S_0^T, R^ S_0^T and the matrices, after which
// the wave that formed L_ab goes on to W; the right-hand sides, X, Y and the
// state update, behind whose MFMAs the next chunk's r, w, k, a, b, v are
// staged in LDS (fp32, w exponentiated for a log-decay input, tokens past the
// end as identity tokens) from registers loaded one chunk earlier. At N = 128 the
// workgroup (eight waves) uses 129 KB of LDS in split form and 111 KB
// otherwise, one per CU; at N = 64 69 KB and 60 KB, two per CU.
//
// MFMA layout (v_mfma_f32_16x16x4_f32): lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; element r of the result is D[4 (l / 16) + r][l % 16].
// The state tile T of a wave holds, in element r of lane l, S[16 w + l % 16]
// [16 T + 4 (l / 16) + r]: the output layout of the update product and the
// B-operand layout of A^ S_0^T when the contraction step (T, r) takes key
// 16 T + 4 g + r from lane group g = l / 16. Products over the 16 tokens take
// token 4 g + s at step s, which is element s of the D layout of X, rhs and Y.
// The bf16 form keeps these layouts: a K = 32 step gives each lane group 8
// elements, standing for keys 16 T + 4 g + e of two key tiles, or for tokens
// 4 g + e with two piece pairs.
#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr float kCfFastMinW = 0x1p-6f;

// SP: the split-bf16 layout (bf16 streams), where the rows that feed the
// state products are also held as bf16 pieces (words of two bf16).
template <int N, bool SP> struct CfLay {
    static constexpr int LD = N + 4;                     // row pitch of [16][N] rows
    static constexpr int TLD = 20;                       // row pitch of [N][16] key-major rows
    static constexpr int MLD = 17;                       // row pitch of 16 x 16 matrices
    static constexpr int PW = N / 2 + 2;                 // words per bf16 row of N keys
    static constexpr int BKW = 50;                       // words per key: per token quad B^ l h m, K^ l h m
    static constexpr int IN = 0;                         // [6][16][LD] r w k a b v
    static constexpr int RWS = SP ? 0 : 16 * LD;         // fp32 rows (fp32 layout only)
    static constexpr int AH = IN + 6 * 16 * LD;          // [16][LD] A^
    static constexpr int RH = AH + RWS;                  // [16][LD] R^
    static constexpr int BH = RH + RWS;                  // [16][LD] B^
    static constexpr int KH = BH + RWS;                  // [16][LD] K^
    static constexpr int BT = KH + RWS;                  // [N][TLD] B^ by key (fp32 layout)
    static constexpr int KT = BT + N * TLD;              // [N][TLD] K^ by key (fp32 layout)
    static constexpr int BK = BT;                        // [N][BKW] words, pieces by key (SP)
    static constexpr int QA = BT + (SP ? N * BKW : 2 * N * TLD);   // [3][16][PW] words, A^ pieces (SP)
    static constexpr int QR = QA + (SP ? 3 * 16 * PW : 0);         // [2][16][PW] words, R^ h and m (SP)
    static constexpr int QB = QR + (SP ? 2 * 16 * PW : 0);         // [3][16][PW] words, B^ / gamma_15 (SP)
    static constexpr int QK = QB + (SP ? 3 * 16 * PW : 0);         // [3][16][PW] words, K^ / gamma_15 (SP)
    static constexpr int MAT = QK + (SP ? 3 * 16 * PW : 0);        // [5][16][MLD] L_ab L_ak M_rb M_rk W
    static constexpr int GAM = MAT + 5 * 16 * MLD;       // [N] gamma_15
    static constexpr int IGAM = GAM + N;                 // [N] 1 / gamma_15 (fast chunks)
    static constexpr int FLAG = IGAM + N;                // [N / 16] per-wave votes
    static constexpr int TOTAL = FLAG + N / 16;
    static_assert(QA % 2 == 0 && QR % 2 == 0 && QB % 2 == 0 && QK % 2 == 0 && GAM % 4 == 0,
                  "8-byte piece rows, 16-byte decay rows");
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
    constexpr bool SP = std::is_same<TI, uint16_t>::value;   // bf16 streams: split-bf16 products
    using L = CfLay<N, SP>;
    constexpr int NT = 4 * N, NW = N / 16, NTILE = N / 16;
    constexpr int WSV = NW >= 8 ? 4 : 0;                 // the wave that forms L_ab and W
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

    // each load's stream is uniform per wave: a select over the kernel's own
    // pointers keeps the loads global (through an array of pointers they
    // become flat loads, which also count against the LDS wait counter)
    const TI *sp[LOADS];
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
        const int s = __builtin_amdgcn_readfirstlane((q * NT + tid) / (16 * GPR));
        const void *vp = s == RR ? p.r : s == RW ? p.w : s == RK ? p.k : s == RA ? p.a : s == RB ? p.b : p.v;
        sp[q] = (const TI *)vp + base;
    }
    Ld16<TI> raw[LOADS];
    auto issue = [&](int c) {
        const int Lc = min(kChunk, u.len - c * kChunk);
        const int64_t t0 = (int64_t)c * kChunk;
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int i = q * NT + tid;
            const int e = (i / GPR) % 16, gq = i % GPR;
            raw[q] = *(const Ld16<TI> *)(sp[q] + (t0 + min(e, Lc - 1)) * ts + gq * EPL);
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
            if (Lc < kChunk && e >= Lc) {                // identity token past the end
#pragma unroll
                for (int k = 0; k < EPL; ++k) x[k] = s == RW ? 1.f : 0.f;
            }
            float *d = sm + L::IN + (s * 16 + e) * L::LD + gq * EPL;
#pragma unroll
            for (int k = 0; k < EPL; k += 4) *(float4 *)(d + k) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
        }
    };
    auto in_at = [&](int s, int t, int j) { return sm[L::IN + (s * 16 + t) * L::LD + j]; };

    if (nch > 0) {
        issue(0);
        stage(0);
        if (nch > 1) issue(1);
    }
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        const int Lc = min(kChunk, u.len - c * kChunk);
        const int64_t t0 = (int64_t)c * kChunk;
        // the state entering the chunk is its checkpoint
        if (p.ckpt) {
            float *ck = p.ckpt + ((u.ckpt + c) * H + h) * (int64_t)(N * N) + (int64_t)row * N + 4 * g;
#pragma unroll
            for (int T = 0; T < NTILE; ++T) *(float4 *)(ck + 16 * T) = make_float4(S[T][0], S[T][1], S[T][2], S[T][3]);
        }
        lds_barrier();                                   // chunk staged; the previous chunk done with LDS
        // ---- prefix and suffix decay products of key j; part 0: A^, gamma_15
        //      and the fast-chunk vote, 1: R^, 2: B^, 3: K^
        {
            const int j = tid % N, part = tid / N;
            // every read of the staged rows first, so that one wait covers them
            const int src = part == 0 ? RA : part == 1 ? RR : part == 2 ? RB : RK;
            float wv[16], xin[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                wv[t] = in_at(RW, t, j);
                xin[t] = in_at(src, t, j);
            }
            bool ok = true;
            // SP: bf16 pieces by token, keys j and j + 1 (j even) in one word:
            // the even lane of the pair writes tokens 0..7, the odd lane
            // tokens 8..15, each taking its partner's value across the pair
            auto token_pieces = [&](const float (&xs)[16], int off, auto npieces) {
                const bool odd = j & 1;
                uint32_t *q = (uint32_t *)(sm + off) + (j >> 1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float mine = odd ? xs[i + 8] : xs[i];
                    const float recv = quad_perm<0xb1>(odd ? xs[i] : xs[i + 8]);
                    const float lo = odd ? recv : mine, hi = odd ? mine : recv;
                    const int t = i + (odd ? 8 : 0);
                    uint32_t ph, pm, pl;
                    split3(lo, hi, ph, pm, pl);
                    q[t * L::PW] = ph;
                    q[(16 + t) * L::PW] = pm;
                    if constexpr (decltype(npieces)::value == 3) q[(32 + t) * L::PW] = pl;
                }
            };
            if (part == 0) {
                float xs[16];
                float gm = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    xs[t] = xin[t] * gm;
                    if constexpr (!SP) sm[L::AH + t * L::LD + j] = xs[t];
                    gm *= wv[t];
                    ok = ok && wv[t] >= kCfFastMinW;
                }
                sm[L::GAM + j] = gm;
                if constexpr (!SP) sm[L::IGAM + j] = 1.f / gm;
                if constexpr (SP) token_pieces(xs, L::QA, std::integral_constant<int, 3>{});
            } else if (part == 1) {
                float xs[16];
                float gm = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    gm *= wv[t];
                    xs[t] = xin[t] * gm;
                    if constexpr (!SP) sm[L::RH + t * L::LD + j] = xs[t];
                }
                if constexpr (SP) token_pieces(xs, L::QR, std::integral_constant<int, 2>{});
            } else {
                float *rowm = sm + (part == 2 ? L::BH : L::KH);
                float *keym = sm + (part == 2 ? L::BT : L::KT) + j * L::TLD;
                float xs[16];
                float sg = 1.f;
#pragma unroll
                for (int s = 15; s >= 0; --s) {
                    xs[s] = xin[s] * sg;
                    if constexpr (!SP) rowm[s * L::LD + j] = xs[s];
                    sg *= wv[s];
                }
                if constexpr (SP) {
                    // bf16 pieces by key, two tokens to a word: for token quad
                    // g, words 12 g .. 12 g + 5 hold B^'s pieces l, h, m (two
                    // words each) and the next six K^'s
                    uint32_t ph[8], pm[8], pl[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) split3(xs[2 * i], xs[2 * i + 1], ph[i], pm[i], pl[i]);
                    uint32_t *q = (uint32_t *)(sm + L::BK) + j * L::BKW + (part == 2 ? 0 : 6);
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        *(u32x2_t *)(q + 12 * gg) = u32x2_t{pl[2 * gg], pl[2 * gg + 1]};
                        *(u32x2_t *)(q + 12 * gg + 2) = u32x2_t{ph[2 * gg], ph[2 * gg + 1]};
                        *(u32x2_t *)(q + 12 * gg + 4) = u32x2_t{pm[2 * gg], pm[2 * gg + 1]};
                    }
                    // and by token, divided by gamma_15 (sg now), for the
                    // matrices of fast chunks (other chunks never read them)
                    const float ig = __builtin_amdgcn_rcpf(sg);   // within 1 ulp (read on fast chunks only)
                    float xt[16];
#pragma unroll
                    for (int t = 0; t < 16; ++t) xt[t] = xs[t] * ig;
                    token_pieces(xt, part == 2 ? L::QB : L::QK, std::integral_constant<int, 3>{});
                } else {
                    // by key: 16-byte stores (a pitch of 20 words puts 8 lanes'
                    // stores on 32 distinct banks; single words would collide 8-way)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(float4 *)(keym + 4 * q) = make_float4(xs[4 * q], xs[4 * q + 1], xs[4 * q + 2], xs[4 * q + 3]);
                }
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
        if constexpr (SP) {
            // A^ S_0^T from six piece products (both operands in three bf16
            // pieces), R^ S_0^T (y only) from the high pieces. A K = 32 MFMA
            // covers the key tiles 2 P and 2 P + 1: element e of lane group g
            // stands for key 16 (2 P + e / 4) + 4 g + e % 4, which is where
            // the state tiles hold them.
            const uint32_t *qa = (const uint32_t *)(sm + L::QA) + l16 * L::PW + 2 * g;
            const uint32_t *qr = (const uint32_t *)(sm + L::QR) + l16 * L::PW + 2 * g;
            f32x4 db = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int P = 0; P < NTILE / 2; ++P) {
                uint32_t h[4], m[4], l[4];
                split3(S[2 * P][0], S[2 * P][1], h[0], m[0], l[0]);
                split3(S[2 * P][2], S[2 * P][3], h[1], m[1], l[1]);
                split3(S[2 * P + 1][0], S[2 * P + 1][1], h[2], m[2], l[2]);
                split3(S[2 * P + 1][2], S[2 * P + 1][3], h[3], m[3], l[3]);
                const u32x4_t sh = {h[0], h[1], h[2], h[3]}, smd = {m[0], m[1], m[2], m[3]},
                              sl = {l[0], l[1], l[2], l[3]};
                auto row8 = [&](const uint32_t *q) {
                    return cat(*(const u32x2_t *)(q + 16 * P), *(const u32x2_t *)(q + 16 * P + 8));
                };
                const u32x4_t ah = row8(qa), am = row8(qa + 16 * L::PW), al = row8(qa + 32 * L::PW);
                da = mfma_bf16_k32(al, sh, da);
                db = mfma_bf16_k32(ah, sl, db);
                da = mfma_bf16_k32(am, smd, da);
                dr = mfma_bf16_k32(row8(qr), sh, dr);
                db = mfma_bf16_k32(am, sh, db);
                da = mfma_bf16_k32(ah, smd, da);
                db = mfma_bf16_k32(ah, sh, db);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) da[r] += db[r];
        } else {
#pragma unroll
            for (int T = 0; T < NTILE; ++T) {
                const float4 a4 = *(const float4 *)(sm + L::AH + l16 * L::LD + 16 * T + 4 * g);
                const float4 r4 = *(const float4 *)(sm + L::RH + l16 * L::LD + 16 * T + 4 * g);
                da = mfma4(a4.x, S[T][0], da); dr = mfma4(r4.x, S[T][0], dr);
                da = mfma4(a4.y, S[T][1], da); dr = mfma4(r4.y, S[T][1], dr);
                da = mfma4(a4.z, S[T][2], da); dr = mfma4(r4.z, S[T][2], dr);
                da = mfma4(a4.w, S[T][3], da); dr = mfma4(r4.w, S[T][3], dr);
            }
        }
        if (fast && SP) {
            // product pm (wave pm % NW): L_ab = A^ (B^ / gamma_15)^T and L_ak
            // from six piece products, M_rb = R^ (B^ / gamma_15)^T and M_rk
            // (y only) from three (two pieces a side: the sums over keys
            // cancel, so one piece a side leaves errors near 1% of y); key
            // slots as in A^ S_0^T
            for (int pm = (wave + NW - WSV) % NW; pm < 4; pm += NW) {
                const uint32_t *qa = (const uint32_t *)(sm + (pm < 2 ? L::QA : L::QR)) + l16 * L::PW + 2 * g;
                const uint32_t *qc = (const uint32_t *)(sm + ((pm & 1) ? L::QK : L::QB)) + l16 * L::PW + 2 * g;
                f32x4 m = {0.f, 0.f, 0.f, 0.f}, m2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int P = 0; P < NTILE / 2; ++P) {
                    auto row8 = [&](const uint32_t *q) {
                        return cat(*(const u32x2_t *)(q + 16 * P), *(const u32x2_t *)(q + 16 * P + 8));
                    };
                    const u32x4_t ah = row8(qa), ch = row8(qc), am = row8(qa + 16 * L::PW),
                                  cm = row8(qc + 16 * L::PW);
                    if (pm < 2) {
                        const u32x4_t al = row8(qa + 32 * L::PW), cl = row8(qc + 32 * L::PW);
                        m = mfma_bf16_k32(al, ch, m);
                        m2 = mfma_bf16_k32(ah, cl, m2);
                        m = mfma_bf16_k32(am, cm, m);
                    }
                    m2 = mfma_bf16_k32(am, ch, m2);
                    m = mfma_bf16_k32(ah, cm, m);
                    m2 = mfma_bf16_k32(ah, ch, m2);
                }
                float *dst = sm + L::MAT + pm * 16 * L::MLD;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * g + r, s = l16;
                    const bool keep = pm < 2 ? s < t : s <= t;
                    dst[t * L::MLD + s] = keep ? m[r] + m2[r] : 0.f;
                }
            }
        } else if (fast) {
            // product pm (wave pm % NW): rows A- (pm < 2) or R-, columns B^ (even) or K^
            for (int pm = (wave + NW - WSV) % NW; pm < 4; pm += NW) {
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
            lds_barrier();                               // (fast is the same on every wave)
        }

        // ---- W = (I - L_ab)^-1 by forward substitution on the wave that
        //      wrote L_ab on fast chunks (once its own LDS writes are done),
        //      after the barrier on other chunks: the quad
        //      of lanes 4 c .. 4 c + 3 owns column c, lane q of it the terms
        //      s = q mod 4 of W[t][c] = [t == c] + sum_{s<t} L_ab[t][s] W[s][c],
        //      completed by a quad sum. The other waves go on to the barrier.
        if (wave == WSV) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
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
        // V is read before the barrier: after it, waves that finish early
        // stage the next chunk over these rows
        float vf[4];                                     // V[token 4 g + s][row]
#pragma unroll
        for (int s = 0; s < 4; ++s) vf[s] = in_at(RV, 4 * g + s, row);
        lds_barrier();

        // ---- rhs = A^ S_0^T + L_ak V (and Y += M_rk V on the fp32 layout)
        // V of bf16 streams is exact in bf16 (one piece)
        const uint32_t vb0 = SP ? pk_bf16(vf[0], vf[1]) : 0u, vb1 = SP ? pk_bf16(vf[2], vf[3]) : 0u;
        const u32x4_t vv = {vb0, vb1, vb0, vb1};
        {
            const float *lak = sm + L::MAT + MLAK * 16 * L::MLD + l16 * L::MLD + 4 * g;
            if constexpr (SP) {
                // L_ak V: L_ak in three pieces; element e of lane group g is
                // token 4 g + e % 4 with piece e / 4 of the pair
                uint32_t h0, m0, l0, h1, m1, l1;
                split3(lak[0], lak[1], h0, m0, l0);
                split3(lak[2], lak[3], h1, m1, l1);
                da = mfma_bf16_k32(u32x4_t{l0, l1, 0u, 0u}, vv, da);
                da = mfma_bf16_k32(u32x4_t{h0, h1, m0, m1}, vv, da);
            } else {
                const float *mrk = sm + L::MAT + MMRK * 16 * L::MLD + l16 * L::MLD + 4 * g;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    da = mfma4(lak[s], vf[s], da);
                    dr = mfma4(mrk[s], vf[s], dr);
                }
            }
        }

        // ---- X = W rhs; Y += M_rb X; y out; S <- S diag(gamma_15) + X^T B^ + V^T K^
        f32x4 xx = {0.f, 0.f, 0.f, 0.f};
        {
            const float *wm = sm + L::MAT + MW * 16 * L::MLD + l16 * L::MLD + 4 * g;
#pragma unroll
            for (int s = 0; s < 4; ++s) xx = mfma4(wm[s], da[s], xx);
            const float *mrb = sm + L::MAT + MMRB * 16 * L::MLD + l16 * L::MLD + 4 * g;
            if constexpr (SP) {
                // y only: M_rb X + M_rk V in one MFMA, one piece each
                const float *mrk = sm + L::MAT + MMRK * 16 * L::MLD + l16 * L::MLD + 4 * g;
                dr = mfma_bf16_k32(u32x4_t{pk_bf16(mrb[0], mrb[1]), pk_bf16(mrb[2], mrb[3]),
                                           pk_bf16(mrk[0], mrk[1]), pk_bf16(mrk[2], mrk[3])},
                                   u32x4_t{pk_bf16(xx[0], xx[1]), pk_bf16(xx[2], xx[3]), vb0, vb1}, dr);
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) dr = mfma4(mrb[s], xx[s], dr);
            }
        }
        if constexpr (SP) {
            // X^T B^ from six piece products, V^T K^ from three (V exact):
            // element e of lane group g is token 4 g + e % 4, piece pair e / 4.
            // A key's row holds, per token quad, B^ pieces l h m then K^
            // pieces l h m, so each A operand is one 16-byte read: (l, h)
            // with (X_h, X_l), (h, m) with (X_h, X_h) and (X_m, X_m), and for
            // K^ (l, h) with (V, 0), (h, m) with (V, V).
            uint32_t xh0, xm0, xl0, xh1, xm1, xl1;
            split3(xx[0], xx[1], xh0, xm0, xl0);
            split3(xx[2], xx[3], xh1, xm1, xl1);
            const u32x4_t xhl = {xh0, xh1, xl0, xl1}, xhh = {xh0, xh1, xh0, xh1}, xmm = {xm0, xm1, xm0, xm1},
                          v0 = {vb0, vb1, 0u, 0u};
#pragma unroll
            for (int T = 0; T < NTILE; ++T) {
                const float4 gm = *(const float4 *)(sm + L::GAM + 16 * T + 4 * g);
                f32x4 acc = f32x4{S[T][0] * gm.x, S[T][1] * gm.y, S[T][2] * gm.z, S[T][3] * gm.w};
                const uint32_t *q = (const uint32_t *)(sm + L::BK) + (16 * T + l16) * L::BKW + 12 * g;
                const u32x4_t blh = *(const u32x4a8_t *)q, bhm = *(const u32x4a8_t *)(q + 2),
                              klh = *(const u32x4a8_t *)(q + 6), khm = *(const u32x4a8_t *)(q + 8);
                acc = mfma_bf16_k32(klh, v0, acc);
                acc = mfma_bf16_k32(blh, xhl, acc);
                acc = mfma_bf16_k32(bhm, xmm, acc);
                acc = mfma_bf16_k32(khm, vv, acc);
                acc = mfma_bf16_k32(bhm, xhh, acc);
                S[T] = acc;
            }
        } else
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
        // ---- stage the next chunk behind the update's MFMAs: every read of
        //      the staged rows came before the last barrier. y leaves after
        //      the staging has waited for its loads: loads and stores share
        //      one wait counter, so stores issued before that wait would hold
        //      it until they are acknowledged.
        if (c + 1 < nch) stage(c + 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            if (t < Lc) IO<TI>::st((TI *)p.y, base + (t0 + t) * ts + row, dr[r]);
        }
        __builtin_amdgcn_sched_barrier(0);               // the stores stay ahead of the loads
        if (c + 2 < nch) issue(c + 2);
    }
    if (p.s_out) {
#pragma unroll
        for (int T = 0; T < NTILE; ++T)
            *(float4 *)(p.s_out + sbase + (int64_t)row * N + 16 * T + 4 * g) = make_float4(S[T][0], S[T][1], S[T][2], S[T][3]);
    }
}

template <typename TI, int N>
hipError_t launch_cf(const FwdArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)(a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B) * a.seg.H;
    const size_t lds = (size_t)CfLay<N, std::is_same<TI, uint16_t>::value>::TOTAL * sizeof(float);
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
