// Gated DeltaNet prefill in chunk form (C = 16) on split-bf16 MFMA, for bf16
// I/O: one workgroup per (sequence, value head), N / 16 waves, wave w holding
// value rows 16 w .. 16 w + 15 of the state in MFMA accumulators.
//
// The gated delta rule S_t = e^{g_t} S_{t-1} (I - beta_t k^_t k^_t^T) +
// beta_t v_t k^_t^T, out_t = S_t q^_t / sqrt(N) is the WKV-7 step with read
// vector q^, decay e^{g_t} on every key, a = -k^, b = beta e^g k^ and written
// key beta k^ (rwkv-lab, "Highlight result -- GDN in RWKV-7"). The chunk form
// of that step (for entering state S_0),
//     X = (I - L_ab)^-1 (A^ S_0^T + L_ak V)
//     Y = R^ S_0^T + M_rb X + M_rk V
//     S_16 = gamma_15 S_0 + X^T B^ + V^T K^
// takes a simple shape because the decay is one scalar per token: with
// E_u = e^{g_u}, gamma_t = prod_{u<=t} E_u and sigma_s = prod_{u>s} E_u,
//     A^_t = -gamma_{t-1} k^_t,  R^_t = gamma_t q^_t,
//     B^_s = beta_s E_s sigma_s k^_s,  K^_s = beta_s sigma_s k^_s,
// and the four 16 x 16 matrices are the Gram matrices k^ k^T and q^ k^T times
// scalar pair decays:
//     L_ab[t][s] = -<k^_t, k^_s> beta_s prod_{s<=u<t} E_u   (s < t)
//     L_ak[t][s] = -<k^_t, k^_s> beta_s prod_{s<u<t} E_u    (s < t)
//     M_rb[t][s] =  <q^_t, k^_s> beta_s prod_{s<=u<=t} E_u  (s <= t)
//     M_rk[t][s] =  <q^_t, k^_s> beta_s prod_{s<u<=t} E_u   (s <= t)
// Every decay factor is a product of E's, never a quotient, so chunks of any
// decay (zero included) take the same path.
//
// Products: A^ S_0^T, L_ak V, X^T B^ and V^T K^ feed the state and take both
// operands in three bf16 pieces (six piece products, fp32 accumulation; v is
// bf16 and takes one); R^ S_0^T and M_rb X + M_rk V feed only the output and
// take one piece; the Gram matrices and X = W rhs are FP32 MFMA. The layouts
// are those of the WKV-7 chunk-form kernel: a K = 32 step gives each lane
// group 8 elements, standing for keys 16 T + 4 g + e of two key tiles, or for
// tokens 4 g + e with two piece pairs.
//
// Per chunk, three LDS barriers: the scaled rows and their pieces (one thread
// per key and row kind); A^ S_0^T, R^ S_0^T, the Gram matrices and the four
// matrices, after which the wave that formed L_ab solves W; the right-hand
// sides, X, Y and the update, behind whose MFMAs the next chunk's q^, k^, v,
// e^g and beta are staged (tokens past the end as identity tokens: q^ = k^ =
// v = 0, e^g = 1, beta = 0). The workgroup uses 73 KB of LDS at N = 128 and
// 40 KB at N = 64. Optionally the state entering each chunk is stored (the
// checkpoints of the GDN backward) and the output skipped.
#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

template <int N> struct GcLay {
    static constexpr int LD = N + 4;                     // row pitch of [16][N] fp32 rows
    static constexpr int MLD = 17;                       // row pitch of 16 x 16 matrices
    static constexpr int PW = N / 2 + 2;                 // words per bf16 row of N keys
    static constexpr int BKW = 50;                       // words per key: per token quad B^ l h m, K^ l h m
    static constexpr int QN = 0;                         // [16][LD] q^
    static constexpr int KN = QN + 16 * LD;              // [16][LD] k^
    static constexpr int VV = KN + 16 * LD;              // [16][LD] v
    static constexpr int EG = VV + 16 * LD;              // [16] e^g
    static constexpr int BE = EG + 16;                   // [16] beta
    static constexpr int BK = BE + 16;                   // [N][BKW] words, B^ and K^ pieces by key
    static constexpr int QA = BK + N * BKW;              // [3][16][PW] words, A^ pieces by token
    static constexpr int QR = QA + 3 * 16 * PW;          // [16][PW] words, R^ high piece
    static constexpr int MAT = QR + 16 * PW;             // [5][16][MLD] L_ab L_ak M_rb M_rk W
    static constexpr int GAM = MAT + 5 * 16 * MLD;       // gamma_15
    static constexpr int TOTAL = GAM + 4;
    static_assert(KN % 4 == 0 && VV % 4 == 0 && EG % 4 == 0 && BK % 2 == 0 && QA % 2 == 0 && QR % 2 == 0,
                  "aligned rows");
};
enum { MLAB = 0, MLAK, MMRB, MMRK, MW };

template <int N>
__global__ __launch_bounds__(4 * N) void gdn_cf_kernel(int32_t T, int32_t H, int32_t Hk,
                                                  const float *__restrict__ qn, const float *__restrict__ kn,
                                                  const uint16_t *__restrict__ v, const float *__restrict__ gg,
                                                  const float *__restrict__ beta, const float *__restrict__ s0,
                                                  uint16_t *__restrict__ out, float *__restrict__ s_out,
                                                  float *__restrict__ ckpt) {
    using L = GcLay<N>;
    constexpr int NW = N / 16, NTILE = N / 16;
    constexpr int WKK = NW >= 8 ? 4 : 0;                 // forms k^ k^T, L_ab, L_ak and W
    constexpr int WQK = WKK + 1;                         // forms q^ k^T, M_rb, M_rk
    extern __shared__ __align__(16) float sm[];

    const int64_t unit = blockIdx.x;                     // b * H + h
    const int h = (int)(unit % H);
    const int64_t b = unit / H;
    const int kh = h / (H / Hk);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const int row = 16 * wave + l16;                     // the lane's value row
    const int64_t sbase = unit * (int64_t)(N * N);
    const int nch = (T + kChunk - 1) / kChunk;
    const float scale = 1.f / sqrtf((float)N);

    // the state: tile T, element r = S[row][16 T + 4 g + r]
    f32x4 S[NTILE];
#pragma unroll
    for (int TT = 0; TT < NTILE; ++TT) {
        S[TT] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s0) {
            const float4 x = *(const float4 *)(s0 + sbase + (int64_t)row * N + 16 * TT + 4 * g);
            S[TT] = f32x4{x.x, x.y, x.z, x.w};
        }
    }

    // loads of a chunk: q^ and k^ float4 tid of [16][N / 4] (every thread);
    // v group tid of [16][N / 8] 16-byte groups (tid < 2 N); e^g's and beta's
    // token (tid - 2 N) and (tid - 2 N - 16) (the next 32 threads). Token rows
    // are clamped into the sequence.
    float4 lq, lk;
    uint4 lv = {0u, 0u, 0u, 0u};
    float lgb = 0.f;
    auto issue = [&](int c) {
        const int t0 = c * kChunk, Lc = min(kChunk, T - t0);
        {
            const int e = tid / (N / 4), c4 = tid % (N / 4);
            const int64_t tok = b * T + t0 + min(e, Lc - 1);
            lq = *(const float4 *)(qn + (tok * Hk + kh) * N + 4 * c4);
            lk = *(const float4 *)(kn + (tok * Hk + kh) * N + 4 * c4);
        }
        if (tid < 2 * N) {
            const int e = tid / (N / 8), c8 = tid % (N / 8);
            const int64_t tok = b * T + t0 + min(e, Lc - 1);
            lv = *(const uint4 *)(v + (tok * H + h) * N + 8 * c8);
        } else if (tid < 2 * N + 16) {
            const int64_t tok = b * T + t0 + min(tid - 2 * N, Lc - 1);
            lgb = gg[tok * H + h];
        } else if (tid < 2 * N + 32) {
            const int64_t tok = b * T + t0 + min(tid - 2 * N - 16, Lc - 1);
            lgb = beta[tok * H + h];
        }
    };
    auto stage = [&](int c) {
        const int Lc = min(kChunk, T - c * kChunk);
        {
            const int e = tid / (N / 4), c4 = tid % (N / 4);
            const bool in = e < Lc;
            *(float4 *)(sm + L::QN + e * L::LD + 4 * c4) = in ? lq : make_float4(0.f, 0.f, 0.f, 0.f);
            *(float4 *)(sm + L::KN + e * L::LD + 4 * c4) = in ? lk : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (tid < 2 * N) {
            const int e = tid / (N / 8), c8 = tid % (N / 8);
            const uint32_t w[4] = {lv.x, lv.y, lv.z, lv.w};
            float x[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[2 * q] = e < Lc ? __uint_as_float(w[q] << 16) : 0.f;
                x[2 * q + 1] = e < Lc ? __uint_as_float(w[q] & 0xffff0000u) : 0.f;
            }
            float *d = sm + L::VV + e * L::LD + 8 * c8;
            *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
            *(float4 *)(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
        } else if (tid < 2 * N + 16) {
            const int e = tid - 2 * N;
            sm[L::EG + e] = e < Lc ? expf(lgb) : 1.f;
        } else if (tid < 2 * N + 32) {
            const int e = tid - 2 * N - 16;
            sm[L::BE + e] = e < Lc ? lgb : 0.f;
        }
    };

    if (nch > 0) {
        issue(0);
        stage(0);
        if (nch > 1) issue(1);
    }
#pragma unroll 1
    for (int c = 0; c < nch; ++c) {
        const int Lc = min(kChunk, T - c * kChunk);
        const int64_t t0 = (int64_t)c * kChunk;
        // the state entering the chunk is its checkpoint (slot b * nch + c)
        if (ckpt) {
            float *ck = ckpt + ((b * nch + c) * H + h) * (int64_t)(N * N) + (int64_t)row * N + 4 * g;
#pragma unroll
            for (int TT = 0; TT < NTILE; ++TT) *(float4 *)(ck + 16 * TT) = make_float4(S[TT][0], S[TT][1], S[TT][2], S[TT][3]);
        }
        lds_barrier();                                   // chunk staged; the previous chunk done with LDS
        // ---- scaled rows of key j; part 0: A^ and gamma_15, 1: R^, 2: B^, 3: K^
        {
            const int j = tid % N, part = tid / N;
            float E[16], xin[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                E[t] = sm[L::EG + t];
                xin[t] = sm[(part == 1 ? L::QN : L::KN) + t * L::LD + j];
            }
            // bf16 pieces by token, keys j and j + 1 (j even) in one word: the
            // even lane of the pair writes tokens 0..7, the odd lane 8..15,
            // each taking its partner's value across the pair
            auto token_pieces = [&](const float (&xs)[16], int off, auto npieces) {
                const bool odd = j & 1;
                uint32_t *q = (uint32_t *)(sm + off) + (j >> 1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float mine = odd ? xs[i + 8] : xs[i];
                    const float recv = quad_perm<0xb1>(odd ? xs[i] : xs[i + 8]);
                    const float lo = odd ? recv : mine, hi = odd ? mine : recv;
                    const int t = i + (odd ? 8 : 0);
                    if constexpr (decltype(npieces)::value == 3) {
                        uint32_t ph, pm, pl;
                        split3(lo, hi, ph, pm, pl);
                        q[t * L::PW] = ph;
                        q[(16 + t) * L::PW] = pm;
                        q[(32 + t) * L::PW] = pl;
                    } else {
                        q[t * L::PW] = pk_bf16(lo, hi);
                    }
                }
            };
            float xs[16];
            if (part == 0) {
                float gm = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    xs[t] = -xin[t] * gm;
                    gm *= E[t];
                }
                if (j == 0) sm[L::GAM] = gm;
                token_pieces(xs, L::QA, std::integral_constant<int, 3>{});
            } else if (part == 1) {
                float gm = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    gm *= E[t];
                    xs[t] = xin[t] * gm;
                }
                token_pieces(xs, L::QR, std::integral_constant<int, 1>{});
            } else {
                float sg = 1.f;
#pragma unroll
                for (int s = 15; s >= 0; --s) {
                    const float f = sm[L::BE + s] * sg;
                    xs[s] = xin[s] * (part == 2 ? f * E[s] : f);
                    sg *= E[s];
                }
                // bf16 pieces by key, two tokens to a word: for token quad gg,
                // words 12 gg .. 12 gg + 5 hold B^'s pieces l, h, m (two words
                // each) and the next six K^'s
                uint32_t ph[8], pm[8], pl[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) split3(xs[2 * i], xs[2 * i + 1], ph[i], pm[i], pl[i]);
                uint32_t *q = (uint32_t *)(sm + L::BK) + j * L::BKW + (part == 2 ? 0 : 6);
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    *(u32x2_t *)(q + 12 * qq) = u32x2_t{pl[2 * qq], pl[2 * qq + 1]};
                    *(u32x2_t *)(q + 12 * qq + 2) = u32x2_t{ph[2 * qq], ph[2 * qq + 1]};
                    *(u32x2_t *)(q + 12 * qq + 4) = u32x2_t{pm[2 * qq], pm[2 * qq + 1]};
                }
            }
        }
        lds_barrier();

        // ---- A^ S_0^T (six piece products) and R^ S_0^T (high pieces, y
        //      only) for the wave's rows, D layout: element r = [token 4 g + r]
        //      [row]. A K = 32 MFMA covers key tiles 2 P and 2 P + 1.
        f32x4 da = {0.f, 0.f, 0.f, 0.f}, dr = {0.f, 0.f, 0.f, 0.f};
        {
            const uint32_t *qa = (const uint32_t *)(sm + L::QA) + l16 * L::PW + 2 * g;
            const uint32_t *qr = (const uint32_t *)(sm + L::QR) + l16 * L::PW + 2 * g;
            f32x4 db = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int P = 0; P < NTILE / 2; ++P) {
                uint32_t hh[4], mm[4], ll[4];
                split3(S[2 * P][0], S[2 * P][1], hh[0], mm[0], ll[0]);
                split3(S[2 * P][2], S[2 * P][3], hh[1], mm[1], ll[1]);
                split3(S[2 * P + 1][0], S[2 * P + 1][1], hh[2], mm[2], ll[2]);
                split3(S[2 * P + 1][2], S[2 * P + 1][3], hh[3], mm[3], ll[3]);
                const u32x4_t sh = {hh[0], hh[1], hh[2], hh[3]}, smd = {mm[0], mm[1], mm[2], mm[3]},
                              sl = {ll[0], ll[1], ll[2], ll[3]};
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
        }
        // ---- the Gram matrix k^ k^T (wave WKK) or q^ k^T (wave WQK) on FP32
        //      MFMA, entry (t = 4 g + r, s = l16) in element r, times the pair
        //      decays: L_ab, L_ak from k^ k^T; M_rb, M_rk from q^ k^T
        if (wave == WKK || wave == WQK) {
            const bool kk = wave == WKK;
            const float *arow = sm + (kk ? L::KN : L::QN) + l16 * L::LD;
            const float *brow = sm + L::KN + l16 * L::LD;
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int TT = 0; TT < NTILE; ++TT) {
                const int j0 = 16 * TT + 4 * g;
                const float4 x4 = *(const float4 *)(arow + j0), y4 = *(const float4 *)(brow + j0);
                m = mfma4(x4.x, y4.x, m);
                m = mfma4(x4.y, y4.y, m);
                m = mfma4(x4.z, y4.z, m);
                m = mfma4(x4.w, y4.w, m);
            }
            const int s = l16;
            const float es = sm[L::EG + s], bs = sm[L::BE + s];
            float E[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) E[u] = sm[L::EG + u];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                float pin = 1.f;                         // prod_{s<u<t} E_u
#pragma unroll
                for (int uu = 0; uu < 16; ++uu) pin *= (uu > s && uu < t) ? E[uu] : 1.f;
                if (kk) {
                    const float lak = s < t ? -m[r] * bs * pin : 0.f;
                    sm[L::MAT + MLAB * 16 * L::MLD + t * L::MLD + s] = lak * es;
                    sm[L::MAT + MLAK * 16 * L::MLD + t * L::MLD + s] = lak;
                } else {
                    const float et = sm[L::EG + t];
                    const float mrk = s <= t ? m[r] * bs * (s < t ? pin * et : 1.f) : 0.f;
                    sm[L::MAT + MMRB * 16 * L::MLD + t * L::MLD + s] = mrk * es;
                    sm[L::MAT + MMRK * 16 * L::MLD + t * L::MLD + s] = mrk;
                }
            }
        }
        // ---- W = (I - L_ab)^-1 by forward substitution on wave WKK, once its
        //      own LDS writes are done: the quad of lanes 4 c .. 4 c + 3 owns
        //      column c, lane q of it the terms s = q mod 4 of W[t][c] =
        //      [t == c] + sum_{s<t} L_ab[t][s] W[s][c], completed by a quad sum
        if (wave == WKK) {
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
                for (int mq = 0; 4 * mq < t; ++mq) lr[t][mq] = lab[t * L::MLD + 4 * mq + qq];
            float wq[4] = {0.f, 0.f, 0.f, 0.f};           // W[4 mq + qq][cc]
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float x = (t == cc && qq == 0) ? 1.f : 0.f;
#pragma unroll
                for (int mq = 0; 4 * mq < t; ++mq) x = fmaf(lr[t][mq], wq[mq], x);
                x = quad_sum(x);
                if ((t & 3) == qq) wq[t >> 2] = x;
            }
#pragma unroll
            for (int mq = 0; mq < 4; ++mq) sm[L::MAT + MW * 16 * L::MLD + (4 * mq + qq) * L::MLD + cc] = wq[mq];
        }
        // v is read before the barrier: after it, waves that finish early
        // stage the next chunk over these rows
        float vf[4];                                     // v[token 4 g + s][row]
#pragma unroll
        for (int s = 0; s < 4; ++s) vf[s] = sm[L::VV + (4 * g + s) * L::LD + row];
        lds_barrier();

        // ---- rhs = A^ S_0^T + L_ak V (L_ak in three pieces, v exact in bf16:
        //      element e of lane group g is token 4 g + e % 4, piece e / 4)
        const uint32_t vb0 = pk_bf16(vf[0], vf[1]), vb1 = pk_bf16(vf[2], vf[3]);
        const u32x4_t vv = {vb0, vb1, vb0, vb1};
        {
            const float *lak = sm + L::MAT + MLAK * 16 * L::MLD + l16 * L::MLD + 4 * g;
            uint32_t h0, m0, l0, h1, m1, l1;
            split3(lak[0], lak[1], h0, m0, l0);
            split3(lak[2], lak[3], h1, m1, l1);
            da = mfma_bf16_k32(u32x4_t{l0, l1, 0u, 0u}, vv, da);
            da = mfma_bf16_k32(u32x4_t{h0, h1, m0, m1}, vv, da);
        }
        // ---- X = W rhs; Y += M_rb X + M_rk V (y only, one piece each); the
        //      update S <- gamma_15 S + X^T B^ + V^T K^
        f32x4 xx = {0.f, 0.f, 0.f, 0.f};
        {
            const float *wm = sm + L::MAT + MW * 16 * L::MLD + l16 * L::MLD + 4 * g;
#pragma unroll
            for (int s = 0; s < 4; ++s) xx = mfma4(wm[s], da[s], xx);
            const float *mrb = sm + L::MAT + MMRB * 16 * L::MLD + l16 * L::MLD + 4 * g;
            const float *mrk = sm + L::MAT + MMRK * 16 * L::MLD + l16 * L::MLD + 4 * g;
            dr = mfma_bf16_k32(u32x4_t{pk_bf16(mrb[0], mrb[1]), pk_bf16(mrb[2], mrb[3]),
                                       pk_bf16(mrk[0], mrk[1]), pk_bf16(mrk[2], mrk[3])},
                               u32x4_t{pk_bf16(xx[0], xx[1]), pk_bf16(xx[2], xx[3]), vb0, vb1}, dr);
        }
        {
            // A key's row holds, per token quad, B^ pieces l h m then K^ pieces
            // l h m: each A operand is one 16-byte read, (l, h) with (X_h, X_l),
            // (h, m) with (X_h, X_h) and (X_m, X_m); for K^ (l, h) with (V, 0),
            // (h, m) with (V, V)
            uint32_t xh0, xm0, xl0, xh1, xm1, xl1;
            split3(xx[0], xx[1], xh0, xm0, xl0);
            split3(xx[2], xx[3], xh1, xm1, xl1);
            const u32x4_t xhl = {xh0, xh1, xl0, xl1}, xhh = {xh0, xh1, xh0, xh1}, xmm = {xm0, xm1, xm0, xm1},
                          v0 = {vb0, vb1, 0u, 0u};
            const float gm = sm[L::GAM];
#pragma unroll
            for (int TT = 0; TT < NTILE; ++TT) {
                f32x4 acc = f32x4{S[TT][0] * gm, S[TT][1] * gm, S[TT][2] * gm, S[TT][3] * gm};
                const uint32_t *q = (const uint32_t *)(sm + L::BK) + (16 * TT + l16) * L::BKW + 12 * g;
                const u32x4_t blh = *(const u32x4a8_t *)q, bhm = *(const u32x4a8_t *)(q + 2),
                              klh = *(const u32x4a8_t *)(q + 6), khm = *(const u32x4a8_t *)(q + 8);
                acc = mfma_bf16_k32(klh, v0, acc);
                acc = mfma_bf16_k32(blh, xhl, acc);
                acc = mfma_bf16_k32(bhm, xmm, acc);
                acc = mfma_bf16_k32(khm, vv, acc);
                acc = mfma_bf16_k32(bhm, xhh, acc);
                S[TT] = acc;
            }
        }
        // ---- stage the next chunk behind the update's MFMAs (every read of
        //      the staged rows came before the last barrier); then the outputs
        //      (loads and stores share one wait counter: stores issued before
        //      the staging's wait would hold it until acknowledged); then the
        //      loads of the chunk after
        if (c + 1 < nch) stage(c + 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            if (out && t < Lc) IO<uint16_t>::st(out, ((b * T + t0 + t) * H + h) * N + row, dr[r] * scale);
        }
        __builtin_amdgcn_sched_barrier(0);               // the stores stay ahead of the loads
        if (c + 2 < nch) issue(c + 2);
    }
    if (s_out) {
#pragma unroll
        for (int TT = 0; TT < NTILE; ++TT)
            *(float4 *)(s_out + sbase + (int64_t)row * N + 16 * TT + 4 * g) =
                make_float4(S[TT][0], S[TT][1], S[TT][2], S[TT][3]);
    }
}

template <int N>
hipError_t launch_n(const GdnFwdArgs &a, hipStream_t stream) {
    const size_t lds = (size_t)GcLay<N>::TOTAL * sizeof(float);
    hipError_t e = hipFuncSetAttribute((const void *)gdn_cf_kernel<N>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_cf_kernel<N>), dim3((unsigned)((int64_t)a.B * a.H)), dim3(4 * N), lds, stream, a.T, a.H,
                       a.Hk, (const float *)a.qn, (const float *)a.kn, (const uint16_t *)a.v, a.g, a.beta, a.s0,
                       (uint16_t *)a.out, a.s_out, a.ckpt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_forward_cf(const GdnFwdArgs &a, hipStream_t stream) {
    return a.N == 128 ? launch_n<128>(a, stream) : launch_n<64>(a, stream);
}

}  // namespace wkv7
