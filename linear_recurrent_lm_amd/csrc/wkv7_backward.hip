// WKV-7 backward, second pass: per-chunk gradients on FP32 MFMA.
//
// Forward recurrence (RWKV-7 WKV-7): S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T
// + v_t k_t^T, y_t = S_t r_t. Gradients of L = sum <dy, y> + <ds_out, S_T>.
// Each chunk starts from its stored checkpoint S_0 (the state entering the
// chunk), dS_C (the gradient of the state leaving it), drhs = W^T dX and W
// (see below); the last three are written by the first pass (the
// state-gradient sweep), which computes them anyway. With these given, chunks are
// independent and run in parallel, kChunksPerGroup consecutive chunks per
// workgroup. Nothing is reconstructed by dividing by w.
//
// Within a chunk the forward is (tokens t = 0..15, as in the forward kernel)
//     X = W (A^ S_0^T + L_ak V),  W = (I - L_ab)^-1
//     Y = R^ S_0^T + M_rb X + M_rk V
//     S_C = S_0 diag(gamma_C) + X^T B^ + V^T K^
// and its reverse mode is
//     dX   = B^ dS_C^T + M_rb^T dY          drhs = W^T dX   (drhs and W from the sweep)
//     dV   = K^ dS_C^T + M_rk^T dY + L_ak^T drhs
//     dA^ = drhs S_0, dR^ = dY S_0, dB^ = X dS_C, dK^ = V dS_C
//     dL_ab = drhs X^T, dL_ak = drhs V^T (strictly lower), dM_rb = dY X^T,
//     dM_rk = dY V^T (lower).
// The 16x16 matrices are built as in the forward: the pairs in different
// 4-token sub-chunks are two 16x16x64 MFMA products D = A_rows B_rows^T of
// rows scaled to shared split points (tokens 8, and 4/12), the pairs inside a
// sub-chunk are dot products of a_t F_ex(t) (r_t F_in(t)) with b_s / F_s. Their
// gradients follow the same split: with dD the matrix gradients gathered in
// the product's index map, dA_rows = dD B_rows and dB_rows = dD^T A_rows (two
// more MFMA products per tile), scaled back by each row's decay factor; the
// within-sub-chunk pairs are short VALU sums.
//
// The decay gradient is assembled as u_m = w_m dw_m, the sum of every decay
// product that contains w_m times its gradient, then dw = u / w. For the
// chunk-level rows these are sums of a_t dA^_t gamma_{t-1} over t > m, of
// r_t dR^_t gamma_t over t >= m, of (b_s dB^_s + k_s dK^_s) D_{15,s} over s < m,
// and dgamma_C gamma_C. For the pairs (t, s) of a split-point block with split
// R, the pairs that contain w_m (s < m <= t for M, s < m < t for L) are, for
// m >= R, all pairs of the rows t >= m: sum_{t >= m} r_t dr_t + sum_{t > m}
// a_t da_t over the block's row gradients; for m < R, all pairs of the columns
// s < m: sum_{s < m} b_s db_s + k_s dk_s over the block's column gradients.
// Pairs inside m's own sub-chunk are summed directly. Every term carries w_m,
// so nothing cancels when w_m is tiny. The backward uses w' = max(w, 2^-30)
// throughout, so dw is finite at w = 0 and equals the gradient there to
// within the clamp.
//
// One 1024-thread workgroup (16 waves) per (sequence, head, chunk group).
// 16x64 chunk matrices and the two 64x64 states live in LDS, row-major; MFMA
// operands are 16-byte loads along the contraction index where the layout
// allows it. Wave w runs on SIMD w % 4; the roles of a phase are spread so
// that the four SIMDs carry similar MFMA and VALU work.
#include <type_traits>

#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr int kThreads = 1024;
constexpr int kChunksPerGroup = 32;               // chunks per workgroup (consecutive)
constexpr int LD = 68;                            // row pitch of 16x64 / 64x64 arrays
constexpr float kMinW = 9.313225746154785e-10f;   // 2^-30

// LDS layout (floats)
constexpr int O_IN = 0;                      // [7][16][LD] r w k a b v dy (w clamped)
constexpr int O_Q = O_IN + 7 * 16 * LD;      // [32][LD] A^ (0..15), R^ (16..31); with B^, K^ later u terms 6..8
constexpr int O_BK = O_Q + 32 * LD;          // [32][LD] B^, K^
constexpr int O_AR = O_BK + 32 * LD;         // [32][LD] A'_t = a_t F_ex(t), R'_t = r_t F_in(t)
constexpr int O_AWR = O_AR + 32 * LD;        // [8][LD]  A'_t W_2, R'_t W_2 for t = 12..15
constexpr int O_BD = O_AWR + 8 * LD;         // [16][LD] b_s / F_s
constexpr int O_KD = O_BD + 16 * LD;         // [16][LD] k_s / F_s
constexpr int O_BL = O_KD + 16 * LD;         // [32][LD] b, k rows scaled to the split points
constexpr int O_S0 = O_BL + 32 * LD;         // [64][LD] S_0; later [4][16][LD] the pair products Z
constexpr int O_DS = O_S0 + 64 * LD;         // [64][LD] dS_C; with X, drhs later u terms 0..5
constexpr int O_X = O_DS + 64 * LD;          // [16][LD] X[t][i]
constexpr int O_DR = O_X + 16 * LD;          // [16][LD] drhs[t][i]
constexpr int O_G = O_DR + 16 * LD;          // [4][16][LD] dA^, dR^, dB^, dK^ ([t][j])
constexpr int O_M = O_G + 64 * LD;           // [11][256] Lab Lak Mrb Mrk W dLab dLak dMrb dMrk dD1 dD2
constexpr int O_GC = O_M + 11 * 256;         // [64] gamma_C
constexpr int O_DGC = O_GC + 64;             // [4][64] d gamma_C, partial sums over 16 rows each
constexpr int O_GO = O_DGC + 4 * 64;         // [6][16][64] 16-bit gradients dv dr da db dk dw of a chunk
constexpr int LDS_FLOATS = O_GO + 6 * 16 * 64 / 2;
static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");

enum { IR = 0, IW, IK, IA, IB, IV, IDY };
// dD1, dD2: the matrix gradients gathered in the index maps of the two
// split-point products (entries outside a map stay zero)
enum { MLAB = 0, MLAK, MMRB, MMRK, MW, MDLAB, MDLAK, MDMRB, MDMRK, MDD1, MDD2 };
enum { ZA1 = 0, ZB1, ZA2, ZB2 };             // pair products: dA_rows, dB_rows of tiles 1, 2
// u terms per token ([16][LD] each): chunk parts a dA^ g, r dR^ g, (b dB^ + k dK^) D;
// block row parts (a da, r dr) of blocks R = 4 / 8 (rows 4..15) and R = 12
// (rows 12..15); block column parts (b db + k dk) of R = 8 (0..7) and R = 4 / 12 (0..3, 8..11)
enum { UCHA = 0, UCHR, UCHC, UR12A, UR12R, UR3A, UR3R, UC2, UC13, kUTerms };

// Products for bf16 streams (SPL): both operands in two bf16 pieces, three
// piece products (h h, h l, l h) on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation, which leaves the VALU free while they run (FP32 MFMAs hold
// it). A K = 32 step gives lane group kq the 8 contraction indices
// k0 + 16 (e / 4) + 4 kq + e % 4, so the output layout is the FP32 one. An
// operand that holds bf16 values (v, dy: AX, BX) is its own high piece, and
// its low piece and that piece's product are skipped. The one-piece form
// (both set for operands that are not bf16 values) rounds each operand to
// bf16 and issues one MFMA per K = 32 step.
template <bool AX, bool BX>
__device__ __forceinline__ f32x4 mm_pieces(f32x4 acc, const float (&a)[8], const float (&b)[8]) {
    uint32_t ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (AX) ah[i] = pk_bf16(a[2 * i], a[2 * i + 1]);
        else split2(a[2 * i], a[2 * i + 1], ah[i], al[i]);
        if constexpr (BX) bh[i] = pk_bf16(b[2 * i], b[2 * i + 1]);
        else split2(b[2 * i], b[2 * i + 1], bh[i], bl[i]);
    }
    const u32x4_t Ah = {ah[0], ah[1], ah[2], ah[3]}, Bh = {bh[0], bh[1], bh[2], bh[3]};
    if constexpr (AX && BX) return mfma_bf16_k32(Ah, Bh, acc);
    f32x4 lo = {0.f, 0.f, 0.f, 0.f};
    if constexpr (!AX) lo = mfma_bf16_k32(u32x4_t{al[0], al[1], al[2], al[3]}, Bh, lo);
    if constexpr (!BX) lo = mfma_bf16_k32(Ah, u32x4_t{bl[0], bl[1], bl[2], bl[3]}, lo);
    acc = mfma_bf16_k32(Ah, Bh, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += lo[r];
    return acc;
}

// acc[m][n] += sum_k A[m][k] B[k][n] with A row-major (pitch lda) and B given
// transposed, Bt[n][k] row-major (pitch ldb): both operands 16-byte loads.
template <int KDIM, bool SPL = false, bool AX = false, bool BX = false>
__device__ __forceinline__ f32x4 mm_AtBt(f32x4 acc, const float *A, int lda, const float *Bt, int ldb,
                                         int l16, int kq) {
    if constexpr (SPL && KDIM % 32 == 0) {
#pragma unroll
        for (int k0 = 0; k0 < KDIM; k0 += 32) {
            const float4 a0 = *(const float4 *)(A + l16 * lda + k0 + 4 * kq);
            const float4 a1 = *(const float4 *)(A + l16 * lda + k0 + 16 + 4 * kq);
            const float4 b0 = *(const float4 *)(Bt + l16 * ldb + k0 + 4 * kq);
            const float4 b1 = *(const float4 *)(Bt + l16 * ldb + k0 + 16 + 4 * kq);
            const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            acc = mm_pieces<AX, BX>(acc, a, b);
        }
        return acc;
    }
#pragma unroll
    for (int k0 = 0; k0 < KDIM; k0 += 16) {
        const float4 a = *(const float4 *)(A + l16 * lda + k0 + 4 * kq);
        const float4 b = *(const float4 *)(Bt + l16 * ldb + k0 + 4 * kq);
        acc = mfma4(a.x, b.x, acc); acc = mfma4(a.y, b.y, acc);
        acc = mfma4(a.z, b.z, acc); acc = mfma4(a.w, b.w, acc);
    }
    return acc;
}

// acc += A B with A row-major (16-byte loads along k) and B row-major [k][n]
// (scalar loads; consecutive lanes read consecutive n).
template <int KDIM, bool SPL = false, bool AX = false, bool BX = false>
__device__ __forceinline__ f32x4 mm_AtB(f32x4 acc, const float *A, int lda, const float *B, int ldb,
                                        int l16, int kq) {
    if constexpr (SPL && KDIM % 32 == 0) {
#pragma unroll
        for (int k0 = 0; k0 < KDIM; k0 += 32) {
            const float4 a0 = *(const float4 *)(A + l16 * lda + k0 + 4 * kq);
            const float4 a1 = *(const float4 *)(A + l16 * lda + k0 + 16 + 4 * kq);
            const float *bp = B + (k0 + 4 * kq) * ldb + l16;
            const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float b[8] = {bp[0], bp[ldb], bp[2 * ldb], bp[3 * ldb],
                                bp[16 * ldb], bp[17 * ldb], bp[18 * ldb], bp[19 * ldb]};
            acc = mm_pieces<AX, BX>(acc, a, b);
        }
        return acc;
    }
#pragma unroll
    for (int k0 = 0; k0 < KDIM; k0 += 16) {
        const float4 a = *(const float4 *)(A + l16 * lda + k0 + 4 * kq);
        const float *bp = B + (k0 + 4 * kq) * ldb + l16;
        acc = mfma4(a.x, bp[0], acc); acc = mfma4(a.y, bp[ldb], acc);
        acc = mfma4(a.z, bp[2 * ldb], acc); acc = mfma4(a.w, bp[3 * ldb], acc);
    }
    return acc;
}

// The 16-bit encoding of a gradient element (round to nearest even).
template <typename TI> __device__ __forceinline__ uint16_t out_bits(float x);
template <> __device__ __forceinline__ uint16_t out_bits<uint16_t>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ uint16_t out_bits<_Float16>(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <> __device__ __forceinline__ uint16_t out_bits<float>(float) { return 0; }   // not used

// acc += sum over 16 indices k = 4 kq + e of a[e] b[e] (this lane's values),
// with b holding bf16 values: one K = 32 MFMA. With a in two bf16 pieces,
// element e of lane group kq is index 4 kq + e % 4, piece e / 4 of a; with
// a rounded to one piece (ONE), elements 4..7 are zero.
template <bool ONE>
__device__ __forceinline__ f32x4 mm_k16_bx(f32x4 acc, const float (&a)[4], const float (&b)[4]) {
    const uint32_t b0 = pk_bf16(b[0], b[1]), b1 = pk_bf16(b[2], b[3]);
    if constexpr (ONE) {
        return mfma_bf16_k32(u32x4_t{pk_bf16(a[0], a[1]), pk_bf16(a[2], a[3]), 0u, 0u},
                             u32x4_t{b0, b1, 0u, 0u}, acc);
    }
    uint32_t h0, l0, h1, l1;
    split2(a[0], a[1], h0, l0);
    split2(a[2], a[3], h1, l1);
    return mfma_bf16_k32(u32x4_t{h0, h1, l0, l1}, u32x4_t{b0, b1, b0, b1}, acc);
}

// acc += sum over 16 indices k = 4 kq + e of a[e] b[e], both rounded to one
// bf16 piece: the FP32 form is four 16x16x4 MFMAs with a[e], b[e] at step e.
__device__ __forceinline__ f32x4 mm_k16_one(f32x4 acc, const float (&a)[4], const float (&b)[4]) {
    return mfma_bf16_k32(u32x4_t{pk_bf16(a[0], a[1]), pk_bf16(a[2], a[3]), 0u, 0u},
                         u32x4_t{pk_bf16(b[0], b[1]), pk_bf16(b[2], b[3]), 0u, 0u}, acc);
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

// Index map of the two split-point products (the forward's tiles): output
// element D[m][n] is the (t, s) entry of L (a rows, isA) or M (r rows), with
// b (isB) or k columns. Tile 1 (split at 8): m < 8 a rows t = 8+m, m >= 8 r
// rows t = m; n < 8 b rows s = n, n >= 8 k rows s = n-8. Tile 2 (splits at 4
// and 12): a rows where m & 4 == 0 with t = 4+m, else r rows t = m; b columns
// where n & 4 == 0 with s = n, else k columns s = n-4; only m, n on the same
// side of 8 are valid.
struct TileEntry { bool valid, isA, isB; int t, s; };
__device__ __forceinline__ TileEntry tile_entry(int tile, int m, int n) {
    TileEntry e;
    if (tile == 0) {
        e.isA = m < 8; e.t = e.isA ? 8 + m : m;
        e.isB = n < 8; e.s = e.isB ? n : n - 8;
        e.valid = true;
    } else {
        e.isA = (m & 4) == 0; e.t = e.isA ? 4 + m : m;
        e.isB = (n & 4) == 0; e.s = e.isB ? n : n - 4;
        e.valid = (m < 8) == (n < 8);
    }
    return e;
}
__device__ __forceinline__ int tile_matrix(const TileEntry &e, int base) {
    return base + (e.isA ? (e.isB ? 0 : 1) : (e.isB ? 2 : 3));   // Lab Lak Mrb Mrk order
}

// The inverse maps: store the gradient v of entry (t, s) of L (isA) or M,
// b (isB) or k column, at its place in dD1 and dD2, if it has one.
__device__ __forceinline__ void tile_scatter(float *sM, bool isA, bool isB, int t, int s, float v) {
    if (t >= 8 && s < 8) sM[MDD1 * 256 + (isA ? t - 8 : t) * 16 + (isB ? s : s + 8)] = v;
    if (((t & 12) == 4 && s < 4) || ((t & 12) == 12 && (s & 12) == 8))
        sM[MDD2 * 256 + (isA ? t - 4 : t) * 16 + (isB ? s : s + 4)] = v;
}

template <int V> struct IC { static constexpr int value = V; };

// Segment mode: the list of the second pass's work items, one per (sequence,
// group of kChunksPerGroup consecutive chunks), so that the launch covers the
// chunks the sequences have rather than ceil(T / 16) chunks for every
// sequence (packed rows are long; most sequences are short). One workgroup:
// each thread counts the groups of a block of sequences, an exclusive scan of
// the counts gives each block its first entry. glist[0] = number of entries
// (at most cap); entry e is (glist[1 + 2e], glist[2 + 2e]) = (sequence, group).
// Invalid table entries count as empty, as in the kernels.
__global__ __launch_bounds__(1024) void group_list_kernel(SegParams seg, int32_t *glist, int64_t cap) {
    __shared__ int64_t part[1024];
    const int tid = threadIdx.x;
    const int n = seg.num_seqs;
    const int per = (n + 1023) / 1024;
    const int s0 = min(n, tid * per), s1 = min(n, s0 + per);
    auto groups = [&](int s) {
        const Unit u = resolve_unit(seg, s);
        const int64_t nch = ((int64_t)u.len + kChunk - 1) / kChunk;
        return (nch + kChunksPerGroup - 1) / kChunksPerGroup;
    };
    int64_t sum = 0;
    for (int s = s0; s < s1; ++s) sum += groups(s);
    part[tid] = sum;
    __syncthreads();
    // inclusive scan of the 1024 block counts (Hillis-Steele)
    for (int d = 1; d < 1024; d <<= 1) {
        const int64_t x = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    int64_t off = part[tid] - sum;
    for (int s = s0; s < s1; ++s) {
        const int64_t gs = groups(s);
        for (int64_t g = 0; g < gs; ++g, ++off) {
            if (off < cap) {
                glist[1 + 2 * off] = s;
                glist[2 + 2 * off] = (int32_t)g;
            }
        }
    }
    if (tid == 1023) glist[0] = (int32_t)(part[1023] < cap ? part[1023] : cap);
}

template <typename TI, bool ONE>
__global__ __launch_bounds__(kThreads, 1) void bwd_chunk_kernel(BwdArgs p, int32_t units) {
    // bf16 streams: every product on bf16 MFMA. With fp32 gradients (ONE
    // false) the K = 64 products take two bf16 pieces a side, within about
    // 2^-16 of the FP32 products, and the K = 16 products of fp32 operands
    // stay on FP32 MFMA. With bf16 gradients (ONE) every operand is rounded
    // to one bf16 piece: the gradients leave in bf16 (2^-9 relative), and
    // the products' own rounding is of that order (measured max per-unit
    // error 6e-3 against the 5e-2 bound, 3e-3 with two pieces).
    constexpr bool kSplitBwd = std::is_same<TI, uint16_t>::value;
    constexpr bool kOne = kSplitBwd && ONE;
    extern __shared__ __align__(16) float sm[];
    // Workgroup -> (unit, group of kChunksPerGroup chunks): dense rows by
    // workgroup index, segment mode through the pre-pass's work list.
    const int H = p.seg.H;
    int h, sq, grp;
    if (p.glist) {
        const int64_t e = blockIdx.x / H;
        h = blockIdx.x % H;
        if (e >= p.glist[0]) return;
        sq = p.glist[1 + 2 * e];
        grp = p.glist[2 + 2 * e];
    } else {
        const int unit = blockIdx.x % units;
        grp = blockIdx.x / units;
        h = unit % H;
        sq = unit / H;
    }
    const Unit u = resolve_unit(p.seg, sq);

    const int tid = threadIdx.x;
    const int lane0 = tid & 63;
    const int wave0 = __builtin_amdgcn_readfirstlane(tid >> 6);  // 16 waves; wave w runs on SIMD w % 4
    int lane = lane0, l16 = lane0 & 15, kq = lane0 >> 4;
    int wave = wave0, w4 = wave0 & 3;                // w4: 16-row / 16-column block of this wave
    // The lane and wave indices are re-derived opaquely at the start of each
    // phase, so that the many LDS addresses and role conditions built from
    // them are formed inside the phase instead of being hoisted out of the
    // chunk loop and kept live (or spilled) throughout.
    auto relane = [&]() {
        int lv = lane0, wv = wave0;
        asm volatile("" : "+v"(lv));
        asm volatile("" : "+s"(wv));
        lane = lv; l16 = lv & 15; kq = lv >> 4;
        wave = wv; w4 = wv & 3;
    };

    float *s_in = sm + O_IN;
    float *s_Q = sm + O_Q, *s_BK = sm + O_BK;
    float *s_AR = sm + O_AR, *s_AWR = sm + O_AWR, *s_BD = sm + O_BD, *s_KD = sm + O_KD, *s_BL = sm + O_BL;
    float *s_S0 = sm + O_S0, *s_DS = sm + O_DS, *s_X = sm + O_X, *s_DR = sm + O_DR;
    float *s_G = sm + O_G, *s_M = sm + O_M, *s_gC = sm + O_GC, *s_dgC = sm + O_DGC;
    float *s_Z = s_S0;                               // reuses S_0 once consumed
    // u terms reuse dS_C, X, drhs (6 arrays) and A^, R^, B^, K^ (3 arrays) once consumed
    auto s_U = [&](int term) { return sm + (term < 6 ? O_DS + term * 16 * LD : O_Q + (term - 6) * 16 * LD); };
    const float *sV = s_in + IV * 16 * LD, *sDY = s_in + IDY * 16 * LD;
    const float *Mlak = s_M + MLAK * 256, *Mmrk = s_M + MMRK * 256;
    const float *Mw = s_M + MW * 256;

    const int64_t ts = (int64_t)H * kN;
    const int64_t base = (u.start * H + h) * kN;
    // gradient stores: the I/O type, or fp32 when requested
    auto gst = [&](void *ptr, int64_t o, float v) {
        if (p.grad_f32) ((float *)ptr)[o] = v;
        else IO<TI>::st((TI *)ptr, o, v);
    };

    const int nch = (u.len + kChunk - 1) / kChunk;
    const int c_lo = grp * kChunksPerGroup;
    const int c_hi = min(nch, c_lo + kChunksPerGroup);
    if (c_lo >= c_hi) return;

    // Upper parts of L_ab, L_ak, M_rb, M_rk and the entries of dD2 outside
    // its index map are never written and stay zero.
    for (int q = tid; q < 4 * 256; q += kThreads) s_M[q] = 0.f;
    for (int q = tid; q < 256; q += kThreads) s_M[MDD2 * 256 + q] = 0.f;

    // Staging: thread tid stages 8 consecutive elements of stream tid / 128
    // (uniform per wave; waves 14, 15 stage none): group g = tid % 128 is
    // token g / 8, elements 8 (g % 8)... Loads are issued one chunk ahead with
    // token rows clamped into the sequence; a missing stream (dy == NULL) is
    // not loaded and stages as zeros.
    Raw<TI, 1> raw;
    float4 ckr, dsr, drr, wwr;                  // checkpoint S_0, dS_C, drhs, W of the chunk in flight
    uint2 dsh, drh;                              // dS_C, drhs in flight as bf16 (kOne: the sweep stores them so)
    const int sst = __builtin_amdgcn_readfirstlane(tid >> 7);
    const TI *ssp = sst < 7 && p.staged[sst] ? (const TI *)p.staged[sst] + base : nullptr;
    // The loads of a chunk are issued in three groups, the inputs in the
    // staging phase and the rest in P3 (waves 0-7) and P5 (waves 8-15), so
    // that the vector-memory instructions of a chunk do not all queue in one
    // phase.
    auto issue_in = [&](int cc) {
        const int Lc = min(kChunk, u.len - cc * kChunk);
        if (ssp) {
            const int g = tid & 127;
            const int t = min(g >> 3, Lc - 1);
            raw_load(ssp + (int64_t)(cc * kChunk) * ts + row_off(t, ts, (g & 7) * 8), raw, 0);
        }
    };
    auto issue_st = [&](int cc) {
        // float4 tid of a 64x64 state: row tid / 16, column 4 (tid % 16)
        const int64_t so = ((u.ckpt + cc) * H + h) * (int64_t)(kN * kN) + tid * 4;
        ckr = *(const float4 *)(p.ckpt + so);
        // drhs [16][64]: float4 tid of waves 0-3; W [16][16]: float4 lane of wave 14
        const int64_t dro = ((u.ckpt + cc) * H + h) * (int64_t)(kChunk * kN) + tid * 4;
        if constexpr (kOne) {
            dsh = *(const uint2 *)((const uint16_t *)p.ws + so);
            if (wave < 4) drh = *(const uint2 *)((const uint16_t *)p.ws_dr + dro);
        } else {
            dsr = *(const float4 *)(p.ws + so);
            if (wave < 4) drr = *(const float4 *)(p.ws_dr + dro);
        }
        if (wave == 14) wwr = *(const float4 *)(p.ws_w + ((u.ckpt + cc) * H + h) * (int64_t)(kChunk * kChunk) + lane * 4);
    };
    issue_in(c_hi - 1);
    issue_st(c_hi - 1);

    // Gradient stores of a chunk are issued during the next chunk, after its
    // staging phase has waited for its loads: loads and stores share one
    // counter, so stores issued just before that wait would hold it until
    // they are acknowledged. 16-bit gradients are gathered in LDS (s_GO) and
    // leave as 16-byte stores, 8 elements per lane, from waves 8-15 in phase
    // P3 (idle there, and before P4 rewrites s_GO); fp32 gradients are held
    // in registers and stored per lane in the staging phase: waves 4-7 hold
    // dv of tokens 4 kq + r at value column 16 (w & 3) + l16, every wave dr,
    // da, db, dk, dw of token w at key column lane.
    const bool wide = !std::is_same<TI, float>::value && !p.grad_f32;
    uint16_t *s_GO = (uint16_t *)(sm + O_GO);
    float pdv[4] = {0.f, 0.f, 0.f, 0.f}, pg[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
    auto flush_wide = [&](int cc) {          // waves 8-15
        const int tc = cc * kChunk, Lc = min(kChunk, u.len - tc);
        // row r of s_GO is gradient r / 16 (uniform per wave), token r % 16;
        // thread f = tid - 512 stores row f / 8 and, on waves 8-11, row 64 + f / 8
        const int f = tid - 512, t = (f >> 3) & 15, c8 = (f & 7) * 8;
        const int g0 = __builtin_amdgcn_readfirstlane(f >> 7);
        auto one = [&](int gi, int row) {
            const uint4 v = *(const uint4 *)(s_GO + row * 64 + c8);
            void *gp = gi == 0 ? p.dv : gi == 1 ? p.dr : gi == 2 ? p.da : gi == 3 ? p.db
                     : gi == 4 ? p.dk : p.dw;
            if (t < Lc) *(uint4 *)((uint16_t *)gp + base + (int64_t)tc * ts + row_off(t, ts, c8)) = v;
        };
        one(g0, f >> 3);
        if (wave < 12) one(4 + g0, 64 + (f >> 3));
    };
    auto flush_regs = [&](int cc) {
        const int tc = cc * kChunk, Lc = min(kChunk, u.len - tc);
        if (wave >= 4 && wave < 8) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * kq + r;
                if (t < Lc) gst(p.dv, base + (int64_t)tc * ts + row_off(t, ts, 16 * w4 + l16), pdv[r]);
            }
        }
        if (wave < Lc) {
            const int64_t o = base + (int64_t)(tc + wave) * ts + lane;
            gst(p.dr, o, pg[0]);
            gst(p.da, o, pg[1]);
            gst(p.db, o, pg[2]);
            gst(p.dk, o, pg[3]);
            gst(p.dw, o, pg[4]);
        }
    };
    // one gradient element of a chunk: into s_GO (16-bit) or the registers
    auto gput = [&](int gi, int t, int col, float v, float &reg) {
        if (wide) s_GO[(gi * 16 + t) * 64 + col] = out_bits<TI>(v);
        else reg = v;
    };

#pragma unroll 1
    for (int c = c_hi - 1; c >= c_lo; --c) {
        const int t0 = c * kChunk;
        const int L = min(kChunk, u.len - t0);
        lds_barrier();
        relane();

        // ---- P0: stage inputs (w clamped; identity tokens past the end), the
        //      checkpoint S_0, dS_C, drhs and W; then prefetch the next chunk's
        //      inputs (and store the previous chunk's fp32 gradients)
        if (sst < 7) {
            const int t = (tid >> 3) & 15, e0 = (tid & 7) * 8;
            float x[8];
            if (ssp) {
                raw_unpack(raw, 0, x);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.f;
            }
            const bool keep = t < L;
            if (sst == IW) {                    // uniform per wave: the clamp only on w
                decay_of<8>(x, p.logw);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = fmaxf(keep ? x[e] : 1.f, kMinW);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = keep ? x[e] : 0.f;
            }
            float *d = s_in + (sst * 16 + t) * LD + e0;
            *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
            *(float4 *)(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
        }
        *(float4 *)(s_S0 + (tid >> 4) * LD + (tid & 15) * 4) = ckr;
        if constexpr (kOne) {
            dsr = make_float4(bf_lo(dsh.x), bf_hi(dsh.x), bf_lo(dsh.y), bf_hi(dsh.y));
            if (wave < 4) drr = make_float4(bf_lo(drh.x), bf_hi(drh.x), bf_lo(drh.y), bf_hi(drh.y));
        }
        *(float4 *)(s_DS + (tid >> 4) * LD + (tid & 15) * 4) = dsr;
        if (wave < 4) *(float4 *)(s_DR + (tid >> 4) * LD + (tid & 15) * 4) = drr;
        if (wave == 14) *(float4 *)(s_M + MW * 256 + lane * 4) = wwr;
        issue_in(max(c - 1, c_lo));
        if (!wide && c < c_hi - 1) flush_regs(c + 1);
        lds_barrier();
        relane();

        // ---- P1: waves 0-7: per-column rows, one role per wave (lane = key
        //      column j), each role reading its inputs before its first store;
        //      waves 8-11: dR^ = dY S_0, waves 12-15: dK^ = V dS_C (key columns
        //      16 (w & 3)..). B^ is not needed (it enters only dX, which comes
        //      from the sweep), so the b rows are split over roles 2 and 6, and
        //      the k rows over roles 3 and 7.
        if (wave < 8) {
            const int role = wave, j = lane;
            const int st = role == 0 || role == 4 ? IA : role == 1 || role == 5 ? IR
                         : role == 2 || role == 6 ? IB : IK;
            float wv[16], xv[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                wv[t] = s_in[(IW * 16 + t) * LD + j];
                xv[t] = s_in[(st * 16 + t) * LD + j];
            }
            if (role == 0) {             // A^_t = a_t gamma_{t-1}; gamma_C
                float g = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) { xv[t] *= g; g *= wv[t]; }
#pragma unroll
                for (int t = 0; t < 16; ++t) s_Q[t * LD + j] = xv[t];
                s_gC[j] = g;
            } else if (role == 1) {      // R^_t = r_t gamma_t
                float g = 1.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) { g *= wv[t]; xv[t] *= g; }
#pragma unroll
                for (int t = 0; t < 16; ++t) s_Q[(16 + t) * LD + j] = xv[t];
            } else if (role == 3) {      // K^_s = k_s D_{15,s}; k_s / F_s
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // 1 / F_s from one reciprocal of the sub-chunk's product
                    // F_{4q+3}, then 1 / F_{s-1} = w_s / F_s going down
                    const float Fq = (wv[4 * q] * wv[4 * q + 1]) * (wv[4 * q + 2] * wv[4 * q + 3]);
                    float inv = __builtin_amdgcn_rcpf(Fq);
#pragma unroll
                    for (int e = 3; e >= 0; --e) {
                        s_KD[(4 * q + e) * LD + j] = xv[4 * q + e] * inv;
                        inv *= wv[4 * q + e];
                    }
                }
                float d = 1.f;
#pragma unroll
                for (int s = 15; s >= 0; --s) { xv[s] *= d; d *= wv[s]; }
#pragma unroll
                for (int s = 0; s < 16; ++s) s_BK[(16 + s) * LD + j] = xv[s];
            } else if (role == 4 || role == 5) {   // A' = a F_ex, R' = r F_in; times W_2 for t >= 12
                const int inc = role - 4;
#pragma unroll
                for (int sc = 0; sc < 4; ++sc) {
                    float f = 1.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 4 * sc + e;
                        if (inc) f *= wv[t];
                        xv[t] *= f;
                        if (!inc) f *= wv[t];
                    }
                }
                const float W2 = (wv[8] * wv[9]) * (wv[10] * wv[11]);
#pragma unroll
                for (int t = 0; t < 16; ++t) s_AR[(16 * inc + t) * LD + j] = xv[t];
#pragma unroll
                for (int e = 0; e < 4; ++e) s_AWR[(4 * inc + e) * LD + j] = xv[12 + e] * W2;
            } else {
                // b rows x_s / F_s (role 2) and scaled to the split points
                // (role 6; B^ itself is not needed); k rows scaled to the
                // split points (role 7; k_s / F_s comes from role 3)
                const int ko = role == 7 ? 1 : 0;
                const bool rows_d = role == 2, rows_l = role != 2;
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
                if (rows_d) {
                    float *dd = ko ? s_KD : s_BD;
#pragma unroll
                    for (int s = 0; s < 16; ++s) dd[s * LD + j] = od[s];
                }
                if (rows_l) {
                    const float W1 = (wv[4] * wv[5]) * (wv[6] * wv[7]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s_BL[(8 * ko + e) * LD + j] = os[e] * W1;          // s = e scaled to 8
                        s_BL[(16 + 4 * ko + e) * LD + j] = os[e];          // s = e scaled to 4
                        s_BL[(8 * ko + 4 + e) * LD + j] = os[4 + e];       // s = 4+e scaled to 8
                        s_BL[(24 + 4 * ko + e) * LD + j] = os[8 + e];      // s = 8+e scaled to 12
                    }
                }
            }
        } else {
            const int jc = 16 * w4;
            const bool isR = wave < 12;
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
            g = mm_AtB<64, kSplitBwd, true, kOne>(g, isR ? sDY : sV, LD, (isR ? s_S0 : s_DS) + jc, LD, l16, kq);
            float *dst = s_G + (isR ? 1 : 3) * 16 * LD + jc + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(4 * kq + r) * LD] = g[r];
        }
        lds_barrier();
        relane();

        // ---- P2: waves 0-3: P_a = A^ S_0^T (value rows 16 w..); waves 4, 5: the
        //      split-point products; waves 6-9: the within-sub-chunk pairs;
        //      waves 10-13: d gamma_C[j] = sum_i dS_C[i][j] S_0[i][j] over rows
        //      16 (w-10)..; wave 14: dM_rk = dY V^T
        f32x4 pa = {0.f, 0.f, 0.f, 0.f};            // waves 0-3 (then rhs, X)
        if (wave < 4) {
            pa = mm_AtBt<64, kSplitBwd, kOne, kOne>(pa, s_Q, LD, s_S0 + 16 * w4 * LD, LD, l16, kq);
        } else if (wave < 6) {
            // the tile index is made a compile-time constant so that the
            // scatter's index map folds
            auto product = [&](auto TILE) {
                constexpr int tile = decltype(TILE)::value;
                const int m = l16;
                const float *arow, *brow;
                if (tile == 0) {
                    arow = m < 4 ? s_AR + (8 + m) * LD : m < 8 ? s_AWR + (m - 4) * LD
                         : m < 12 ? s_AR + (16 + m) * LD : s_AWR + (m - 8) * LD;
                    brow = s_BL + l16 * LD;
                } else {
                    arow = s_AR + ((m & 4) ? 16 + m : 4 + m) * LD;
                    brow = s_BL + (16 + l16) * LD;
                }
                const f32x4 d = kSplitBwd ? mm_AtBt<64, true, kOne, kOne>(f32x4{0.f, 0.f, 0.f, 0.f}, arow, 0, brow, 0, 0, kq)
                                          : rows_product(arow, brow, kq);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const TileEntry e = tile_entry(tile, 4 * kq + r, l16);
                    // L_ak and M_rk only: L_ab and M_rb enter only W and dX,
                    // which come from the sweep
                    if (e.valid && !e.isB) s_M[tile_matrix(e, MLAB) * 256 + e.t * 16 + e.s] = d[r];
                }
            };
            if (wave == 4) product(IC<0>{});
            else product(IC<1>{});
        } else if (wave < 10) {
            // 64 items (sub-chunk p, pair k) x 4 quarters of the 64 columns
            // = 256 units, one per lane of waves 6-9
            const int unit_ = (wave - 6) * 64 + lane;
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
            const float *ar = s_AR + ((isL ? 0 : 16) + t) * LD + 16 * qtr;
            const float *kd = s_KD + s * LD + 16 * qtr;
            float k_ = 0.f;
#pragma unroll
            for (int jj = 0; jj < 16; jj += 4) {
                const float4 x = *(const float4 *)(ar + jj);
                const float4 k4 = *(const float4 *)(kd + jj);
                k_ = fmaf(x.x, k4.x, k_); k_ = fmaf(x.y, k4.y, k_);
                k_ = fmaf(x.z, k4.z, k_); k_ = fmaf(x.w, k4.w, k_);
            }
            k_ = quad_sum(k_);
            if ((lane & 3) == 0) s_M[(isL ? MLAK : MMRK) * 256 + t * 16 + s] = k_;
        } else if (wave < 14) {
            const int j = lane, i0 = 16 * (wave - 10);
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int i = i0; i < i0 + 16; i += 2) {
                acc0 = fmaf(s_DS[i * LD + j], s_S0[i * LD + j], acc0);
                acc1 = fmaf(s_DS[(i + 1) * LD + j], s_S0[(i + 1) * LD + j], acc1);
            }
            s_dgC[(wave - 10) * 64 + j] = acc0 + acc1;
        } else if (wave == 14) {
            f32x4 gm = {0.f, 0.f, 0.f, 0.f};
            gm = mm_AtBt<64, kSplitBwd, true, true>(gm, sDY, LD, sV, LD, l16, kq);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * kq + r;
                const float v = l16 <= t ? gm[r] : 0.f;
                s_M[MDMRK * 256 + t * 16 + l16] = v;
                tile_scatter(s_M, false, false, t, l16, v);
            }
        }
        lds_barrier();
        relane();

        // ---- P3: waves 0-3: rhs = P_a + L_ak V, then X = W rhs (value rows
        //      16 w..) into LDS (W of the chunk was staged from the sweep's
        //      output); waves 4-7: dV partial = K^ dS_C^T + M_rk^T dY (value
        //      rows 16 (w-4)..); waves 8-15: the previous chunk's 16-bit
        //      gradient stores. Then waves 0-7 issue their part of the next
        //      chunk's loads of S_0, dS_C, drhs and W (waves 8-15 in P5).
        f32x4 dvp = {0.f, 0.f, 0.f, 0.f};           // waves 4-7
        if (wave < 4) {
            if constexpr (kSplitBwd) {                 // L_ak V, v holding bf16 values
                const float4 m4 = *(const float4 *)(Mlak + l16 * 16 + 4 * kq);
                const float *vp = sV + 16 * w4 + 4 * kq * LD + l16;
                const float am[4] = {m4.x, m4.y, m4.z, m4.w}, bv[4] = {vp[0], vp[LD], vp[2 * LD], vp[3 * LD]};
                pa = mm_k16_bx<kOne>(pa, am, bv);
            } else {
                pa = mm_AtB<16>(pa, Mlak, 16, sV + 16 * w4, LD, l16, kq);
            }
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            const float4 wr = *(const float4 *)(Mw + l16 * 16 + 4 * kq);
            if constexpr (kOne) {
                o = mm_k16_one(o, {wr.x, wr.y, wr.z, wr.w}, {pa[0], pa[1], pa[2], pa[3]});
            } else {
                o = mfma4(wr.x, pa[0], o); o = mfma4(wr.y, pa[1], o);
                o = mfma4(wr.z, pa[2], o); o = mfma4(wr.w, pa[3], o);
            }
            float *dst = s_X + 16 * w4 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(4 * kq + r) * LD] = o[r];
        } else if (wave < 8) {
            const int i0 = 16 * w4;
            dvp = mm_AtBt<64, kSplitBwd, kOne, kOne>(dvp, s_BK + 16 * LD, LD, s_DS + i0 * LD, LD, l16, kq);
            if constexpr (kSplitBwd) {                 // M_rk^T dY, dy holding bf16 values
                float am[4], bv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    am[e] = Mmrk[(4 * kq + e) * 16 + l16];
                    bv[e] = sDY[(4 * kq + e) * LD + i0 + l16];
                }
                dvp = mm_k16_bx<kOne>(dvp, am, bv);
            } else {
                dvp = mm_TB(dvp, Mmrk, 16, sDY + i0, LD, l16, kq);
            }
        } else if (wide && c < c_hi - 1) {
            flush_wide(c + 1);
        }
        if (wave < 8) issue_st(max(c - 1, c_lo));
        lds_barrier();
        relane();

        // dL_ab = drhs X^T, dL_ak = drhs V^T, dM_rb = dY X^T (mi = 0, 1, 2),
        // with their scatter into the index maps of the split-point products;
        // the matrix index is a compile-time constant so that the scatter's
        // index maps fold
        auto dlm_product = [&](auto MI) {
            constexpr int mi = decltype(MI)::value;
            const float *lhs = mi < 2 ? s_DR : sDY;
            const float *rt = mi == 1 ? sV : s_X;
            f32x4 gm = {0.f, 0.f, 0.f, 0.f};
            gm = mm_AtBt<64, kSplitBwd, mi == 2 || kOne, mi == 1 || kOne>(gm, lhs, LD, rt, LD, l16, kq);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * kq + r;
                const bool keep = mi < 2 ? (l16 < t) : (l16 <= t);
                const float v = keep ? gm[r] : 0.f;
                s_M[(MDLAB + mi) * 256 + t * 16 + l16] = v;
                tile_scatter(s_M, mi < 2, mi != 1, t, l16, v);
            }
        };

        // ---- P4: waves 4-7 finish dV = partial + L_ak^T drhs (held for the
        //      store); waves 0-3: dA^ = drhs S_0 (key columns 16 (w & 3)..);
        //      waves 12, 13, 14: dL_ab, dL_ak, dM_rb
        if (wave >= 4 && wave < 8) {
            const int i0 = 16 * w4;
            float am[4], bm[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                am[e] = Mlak[(4 * kq + e) * 16 + l16];
                bm[e] = s_DR[(4 * kq + e) * LD + i0 + l16];
            }
            if constexpr (kOne) {
                dvp = mm_k16_one(dvp, am, bm);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) dvp = mfma4(am[e], bm[e], dvp);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) gput(0, 4 * kq + r, i0 + l16, dvp[r], pdv[r]);
        } else if (wave < 4) {
            const int jc = 16 * w4;
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
            g = mm_AtB<64, kSplitBwd, kOne, kOne>(g, s_DR, LD, s_S0 + jc, LD, l16, kq);
            float *dst = s_G + jc + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(4 * kq + r) * LD] = g[r];
        } else if (wave == 12) {
            dlm_product(IC<0>{});
        } else if (wave == 13) {
            dlm_product(IC<1>{});
        } else if (wave == 14) {
            dlm_product(IC<2>{});
        }
        lds_barrier();
        relane();

        // ---- P5: pair-gradient products of the split-point tiles (waves 0-3):
        //      Z_A = dD B_rows and Z_B = dD^T A_rows of tiles 1, 2 (wave w:
        //      Z_A1, Z_B1, Z_A2, Z_B2), all 64 columns; into s_Z (S_0 is consumed).
        //      Waves 8-11: dB^ = X dS_C; waves 8-15: their part of the next
        //      chunk's loads
        if (wave < 4) {
            const int prod = wave;
            const int tile = prod >> 1;
            const bool zb = (prod & 1) != 0;
            const float *dD = s_M + (MDD1 + tile) * 256;
            float av[4];
            const float *brow[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                av[e] = dD[zb ? (4 * kq + e) * 16 + l16 : l16 * 16 + 4 * kq + e];
                const int r_ = 4 * kq + e;
                if (!zb) {
                    brow[e] = s_BL + (tile == 0 ? r_ : 16 + r_) * LD;
                } else if (tile == 0) {
                    brow[e] = r_ < 4 ? s_AR + (8 + r_) * LD : r_ < 8 ? s_AWR + (r_ - 4) * LD
                            : r_ < 12 ? s_AR + (16 + r_) * LD : s_AWR + (r_ - 8) * LD;
                } else {
                    brow[e] = s_AR + ((r_ & 4) ? 16 + r_ : 4 + r_) * LD;
                }
            }
            float bv[4][4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[q][e] = brow[e][16 * q + l16];
            float *zo = s_Z + prod * 16 * LD + l16;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                if constexpr (kOne) {
                    z = mm_k16_one(z, av, bv[q]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) z = mfma4(av[e], bv[q][e], z);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) zo[(4 * kq + r) * LD + 16 * q] = z[r];
            }
        } else if (wave >= 8) {
            if (wave < 12) {          // dB^ = X dS_C (key columns 16 (w & 3)..)
                const int jc = 16 * w4;
                f32x4 g = {0.f, 0.f, 0.f, 0.f};
                g = mm_AtB<64, kSplitBwd, kOne, kOne>(g, s_X, LD, s_DS + jc, LD, l16, kq);
                float *dst = s_G + 2 * 16 * LD + jc + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(4 * kq + r) * LD] = g[r];
            }
            issue_st(max(c - 1, c_lo));
        }
        lds_barrier();
        relane();

        // ---- P6a: per-token gradients of key column j = lane for token t = w
        //      (token bodies specialised at compile time): chunk parts,
        //      split-point pair parts (Z scaled by the decay factors) and
        //      within-sub-chunk pair parts give dr, da, db, dk (stored); the u
        //      terms go to LDS (dS_C, X, drhs, A^..K^ are consumed)
        {
            const int j = lane;
            float wv[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) wv[t] = s_in[(IW * 16 + t) * LD + j];
            const float W1 = (wv[4] * wv[5]) * (wv[6] * wv[7]);
            const float W2 = (wv[8] * wv[9]) * (wv[10] * wv[11]);
            const float *dLab = s_M + MDLAB * 256, *dLak = s_M + MDLAK * 256;
            const float *dMrb = s_M + MDMRB * 256, *dMrk = s_M + MDMRK * 256;
            auto tok = [&](auto TT) {
                constexpr int t = decltype(TT)::value;
                constexpr int p0 = t & ~3;                    // first token of t's sub-chunk
                // decay factors of column j at token t
                // each product is one left-to-right chain; gam, fin and dend
                // extend gprev, fex and suf
                float gprev = 1.f, fex = 1.f, suf = 1.f;
#pragma unroll
                for (int u2 = 0; u2 < t; ++u2) gprev *= wv[u2];
#pragma unroll
                for (int u2 = p0; u2 < t; ++u2) fex *= wv[u2];
#pragma unroll
                for (int u2 = t + 1; u2 < p0 + 4; ++u2) suf *= wv[u2];
                const float gam = gprev * wv[t], fin = fex * wv[t];
                float dend = suf;
#pragma unroll
                for (int u2 = p0 + 4; u2 < 16; ++u2) dend *= wv[u2];
                const float invF = __builtin_amdgcn_rcpf(fin);
                const float *zA1 = s_Z + ZA1 * 16 * LD + j, *zB1 = s_Z + ZB1 * 16 * LD + j;
                const float *zA2 = s_Z + ZA2 * 16 * LD + j, *zB2 = s_Z + ZB2 * 16 * LD + j;
                // split-point pair parts by block: rows of block R = 8 (t >= 8) and
                // of R = 4 / 12 (t in 4..7 / 12..15); columns of R = 8 (s < 8) and
                // of R = 4 / 12 (s in 0..3 / 8..11)
                float a8 = 0.f, r8 = 0.f, a4 = 0.f, r4 = 0.f, b8 = 0.f, k8 = 0.f, b4 = 0.f, k4 = 0.f;
                if (t >= 8) {
                    const float sc = t >= 12 ? W2 : 1.f;
                    a8 = fex * zA1[(t - 8) * LD] * sc;
                    r8 = fin * zA1[t * LD] * sc;
                }
                if ((t & 4) != 0) {
                    a4 = fex * zA2[(t - 4) * LD];
                    r4 = fin * zA2[t * LD];
                }
                if (t < 8) {
                    const float sc = t < 4 ? W1 : 1.f;
                    b8 = suf * zB1[t * LD] * sc;
                    k8 = suf * zB1[(8 + t) * LD] * sc;
                }
                if ((t & 4) == 0 && t < 12) {
                    b4 = suf * zB2[t * LD];
                    k4 = suf * zB2[(t + 4) * LD];
                }
                // within-sub-chunk pair parts: t as the row (s <= t) and as the
                // column (rows s >= t of M, s > t of L)
                float qa = 0.f, qr = 0.f, qb = 0.f, qk = 0.f;
#pragma unroll
                for (int s = p0; s < p0 + 4; ++s) {
                    if (s <= t) {
                        const float bd = s_BD[s * LD + j], kd = s_KD[s * LD + j];
                        if (s < t) qa += dLab[t * 16 + s] * bd + dLak[t * 16 + s] * kd;
                        qr += dMrb[t * 16 + s] * bd + dMrk[t * 16 + s] * kd;
                    }
                    if (s >= t) {
                        const float rp = s_AR[(16 + s) * LD + j];
                        qb += dMrb[s * 16 + t] * rp;
                        qk += dMrk[s * 16 + t] * rp;
                    }
                    if (s > t) {
                        const float ap = s_AR[s * LD + j];
                        qb += dLab[s * 16 + t] * ap;
                        qk += dLak[s * 16 + t] * ap;
                    }
                }
                const float a_t = s_in[(IA * 16 + t) * LD + j], r_t = s_in[(IR * 16 + t) * LD + j];
                const float b_t = s_in[(IB * 16 + t) * LD + j], k_t = s_in[(IK * 16 + t) * LD + j];
                const float dAh = s_G[(0 * 16 + t) * LD + j], dRh = s_G[(1 * 16 + t) * LD + j];
                const float dBh = s_G[(2 * 16 + t) * LD + j], dKh = s_G[(3 * 16 + t) * LD + j];
                const float dac = dAh * gprev, drc = dRh * gam, dbc = dBh * dend, dkc = dKh * dend;
                gput(1, t, j, drc + fin * qr + r8 + r4, pg[0]);
                gput(2, t, j, dac + fex * qa + a8 + a4, pg[1]);
                gput(3, t, j, dbc + invF * qb + b8 + b4, pg[2]);
                gput(4, t, j, dkc + invF * qk + k8 + k4, pg[3]);
                // u terms that the scans below read (ranges with structural zeros
                // are neither written nor read)
                const int o = t * LD + j;
                s_U(UCHA)[o] = a_t * dac;
                s_U(UCHR)[o] = r_t * drc;
                s_U(UCHC)[o] = b_t * dbc + k_t * dkc;
                if (t >= 4) {
                    s_U(UR12A)[o] = a_t * (a8 + (t >= 12 ? 0.f : a4));
                    s_U(UR12R)[o] = r_t * (r8 + (t >= 12 ? 0.f : r4));
                }
                if (t >= 12) {
                    s_U(UR3A)[o] = a_t * a4;
                    s_U(UR3R)[o] = r_t * r4;
                }
                if (t < 8) s_U(UC2)[o] = b_t * b8 + k_t * k8;
                if ((t & 4) == 0 && t < 12) s_U(UC13)[o] = b_t * b4 + k_t * k4;
            };
            switch (wave) {
                case 0: tok(IC<0>{}); break;
                case 1: tok(IC<1>{}); break;
                case 2: tok(IC<2>{}); break;
                case 3: tok(IC<3>{}); break;
                case 4: tok(IC<4>{}); break;
                case 5: tok(IC<5>{}); break;
                case 6: tok(IC<6>{}); break;
                case 7: tok(IC<7>{}); break;
                case 8: tok(IC<8>{}); break;
                case 9: tok(IC<9>{}); break;
                case 10: tok(IC<10>{}); break;
                case 11: tok(IC<11>{}); break;
                case 12: tok(IC<12>{}); break;
                case 13: tok(IC<13>{}); break;
                case 14: tok(IC<14>{}); break;
                default: tok(IC<15>{}); break;
            }
        }
        lds_barrier();
        relane();

        // ---- P6b: per key column j = lane, the partial sums of u_m for all m
        //      (each a prefix or suffix sum over one block's range, so no sum
        //      is formed as a difference): wave 0 chunk rows (t >= m for r,
        //      t > m for a), wave 1 chunk columns (s < m), wave 2 block rows,
        //      wave 3 block columns, waves 4-7 the pairs of sub-chunk w-4 that
        //      straddle m. Results [5][16][LD] into s_Z (4) and s_G (1).
        {
            const int j = lane;
            const float *dLab = s_M + MDLAB * 256, *dLak = s_M + MDLAK * 256;
            const float *dMrb = s_M + MDMRB * 256, *dMrk = s_M + MDMRK * 256;
            if (wave == 0) {
                float rr[16], aa[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) { rr[t] = s_U(UCHR)[t * LD + j]; aa[t] = s_U(UCHA)[t * LD + j]; }
                float acc = 0.f;
#pragma unroll
                for (int t = 15; t >= 0; --t) { s_Z[t * LD + j] = acc + rr[t]; acc += rr[t] + aa[t]; }
            } else if (wave == 1) {
                float cc[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) cc[t] = s_U(UCHC)[t * LD + j];
                float acc = 0.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) { s_Z[(16 + t) * LD + j] = acc; acc += cc[t]; }
            } else if (wave == 2) {
                // block R = 8 rows t = 8..15 (with R = 12 rows t = 12..15 once
                // m >= 12); block R = 4 rows t = 4..7
                float rr[16], aa[16], r3[16], a3[16];
#pragma unroll
                for (int t = 4; t < 16; ++t) { rr[t] = s_U(UR12R)[t * LD + j]; aa[t] = s_U(UR12A)[t * LD + j]; }
#pragma unroll
                for (int t = 12; t < 16; ++t) { r3[t] = s_U(UR3R)[t * LD + j]; a3[t] = s_U(UR3A)[t * LD + j]; }
                float *res = s_Z + 2 * 16 * LD + j;
                float acc = 0.f, acc3 = 0.f;
#pragma unroll
                for (int t = 15; t >= 12; --t) {
                    res[t * LD] = acc + acc3 + rr[t] + r3[t];
                    acc += rr[t] + aa[t]; acc3 += r3[t] + a3[t];
                }
#pragma unroll
                for (int t = 11; t >= 8; --t) { res[t * LD] = acc + rr[t]; acc += rr[t] + aa[t]; }
                acc = 0.f;
#pragma unroll
                for (int t = 7; t >= 4; --t) { res[t * LD] = acc + rr[t]; acc += rr[t] + aa[t]; }
#pragma unroll
                for (int t = 0; t < 4; ++t) res[t * LD] = 0.f;
            } else if (wave == 3) {
                // block R = 8 columns s = 0..7, R = 4 columns s = 0..3, R = 12 columns s = 8..11
                float c2[8], c13[12];
#pragma unroll
                for (int t = 0; t < 8; ++t) c2[t] = s_U(UC2)[t * LD + j];
#pragma unroll
                for (int t = 0; t < 12; ++t)
                    if ((t & 4) == 0) c13[t] = s_U(UC13)[t * LD + j];
                float *res = s_Z + 3 * 16 * LD + j;
                float acc = 0.f, acc13 = 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t) { res[t * LD] = acc + acc13; acc += c2[t]; acc13 += c13[t]; }
#pragma unroll
                for (int t = 4; t < 8; ++t) { res[t * LD] = acc; acc += c2[t]; }
                acc = 0.f;
#pragma unroll
                for (int t = 8; t < 12; ++t) { res[t * LD] = acc; acc += c13[t]; }
#pragma unroll
                for (int t = 12; t < 16; ++t) res[t * LD] = 0.f;
            } else if (wave < 8) {
                // pairs (p0+tt, p0+ss), ss < tt, inside sub-chunk p0 = 4(w-4):
                // M pairs contain w_m for ss < m-p0 <= tt, L pairs for ss < m-p0 < tt
                const int p0 = 4 * (wave - 4);
                float ap[4], rp[4], bd[3], kd[3];
#pragma unroll
                for (int e = 1; e < 4; ++e) {
                    ap[e] = s_AR[(p0 + e) * LD + j];
                    rp[e] = s_AR[(16 + p0 + e) * LD + j];
                }
#pragma unroll
                for (int e = 0; e < 3; ++e) { bd[e] = s_BD[(p0 + e) * LD + j]; kd[e] = s_KD[(p0 + e) * LD + j]; }
                float pm[4][3], pl[4][3];
#pragma unroll
                for (int tt = 1; tt < 4; ++tt)
#pragma unroll
                    for (int ss = 0; ss < tt; ++ss) {
                        const int o = (p0 + tt) * 16 + p0 + ss;
                        pm[tt][ss] = rp[tt] * (dMrb[o] * bd[ss] + dMrk[o] * kd[ss]);
                        pl[tt][ss] = ap[tt] * (dLab[o] * bd[ss] + dLak[o] * kd[ss]);
                    }
                float *res = s_G + j;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    float x = 0.f;
#pragma unroll
                    for (int tt = mi; tt < 4; ++tt)
#pragma unroll
                        for (int ss = 0; ss < mi; ++ss) {
                            x += pm[tt][ss];
                            if (tt > mi) x += pl[tt][ss];
                        }
                    res[(p0 + mi) * LD] = x;
                }
            }
        }
        lds_barrier();
        relane();

        // ---- P6c: u_m for m = w: the five partial sums and d gamma_C gamma_C;
        //      dw = u / w (stored with the other gradients of the chunk)
        {
            const int j = lane, m = wave;
            const int o = m * LD + j;
            const float dgc = (s_dgC[j] + s_dgC[64 + j]) + (s_dgC[128 + j] + s_dgC[192 + j]);
            const float x = dgc * s_gC[j] + ((s_Z[o] + s_Z[16 * LD + o]) + (s_Z[32 * LD + o] + s_Z[48 * LD + o]))
                          + s_G[o];
            // d/dw = u / w (v_rcp_f32, within 1 ulp); for a log-decay input
            // d/d log(w) = u itself
            gput(5, m, j, p.logw ? x : x * __builtin_amdgcn_rcpf(s_in[IW * 16 * LD + o]), pg[4]);
        }
    }
    lds_barrier();
    relane();
    if (wide) {
        if (wave >= 8) flush_wide(c_lo);
    } else {
        flush_regs(c_lo);
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
    // bf16 streams: one-piece products for bf16 gradients, two pieces for fp32 ones
    auto fn = a.dtype == 1 ? (a.grad_f32 ? bwd_chunk_kernel<uint16_t, false> : bwd_chunk_kernel<uint16_t, true>)
            : a.dtype == 2 ? bwd_chunk_kernel<_Float16, false> : bwd_chunk_kernel<float, false>;
    hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (a.seg.num_seqs > 0 && a.glist) {
        // work items from the segment table: at most ceil(slots / 8) + num_seqs
        hipLaunchKernelGGL(group_list_kernel, dim3(1), dim3(1024), 0, stream, a.seg, a.glist, a.glist_cap);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fn, dim3((unsigned)(a.glist_cap * a.seg.H)), dim3(kThreads), lds, stream, a, units);
        return hipGetLastError();
    }
    // A row has ceil(T / 16) chunks.
    a.glist = nullptr;
    const int max_chunks = (a.seg.T + kChunk - 1) / kChunk;
    const int64_t groups = (max_chunks + kChunksPerGroup - 1) / kChunksPerGroup;
    hipLaunchKernelGGL(fn, dim3((unsigned)(groups * units)), dim3(kThreads), lds, stream, a, units);
    return hipGetLastError();
}

}  // namespace wkv7
