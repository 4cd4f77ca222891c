// Linear-head cross-entropy over a large vocabulary, streamed over the
// vocabulary (rwkv-metal, "Open problems / contributions welcome": an online
// softmax in the forward, softmax-form gradients in the backward; rwkv-lab,
// "From-scratch pretraining lab": fused LM-head cross-entropy with pad
// masking). For hidden rows h[m] (D wide), head rows W[v] and targets t_m:
//     z[m, v] = <h[m], W[v]>,  lse[m] = log sum_v exp z[m, v],
//     loss[m] = lse[m] - z[m, t_m],  G = dloss (softmax - onehot),
//     dh = G W,  dW = G^T h;  rows with t_m outside [0, V) are pad rows.
//
// One bf16 MFMA GEMM core, C[i][j] = sum_k A[i][k] B[j][k] with both operands
// contiguous along k, serves every product through its epilogue:
//   FWD   A = W, B = h: logits^T tiles (vocabulary down, tokens across). Each
//         lane keeps a running (max, sum of exp) for its token columns over
//         the vocabulary tiles of its split, in base-2 units; the target
//         logit is taken from the tile that holds it. The [M, V] logits are
//         never stored; a small kernel merges the splits into lse and loss.
//   GRAD  the same tiles recomputed for one chunk of vocabulary rows: G =
//         dloss (2^(z log2 e - lse log2 e) - [v == t]) rounded to bf16 and
//         stored twice, G [m][v] (contiguous along v, for dh) and G^T [v][m]
//         (contiguous along m, for dW). The chunk bounds the memory to
//         M x chunk.
//   STORE dW rows of the chunk = G^T (h^T)^T, written once, and dh += G
//         (W^T)^T, with W^T and h^T transposed copies padded with zeros, so
//         that every product contracts along a contiguous, 64-aligned
//         dimension. Chunking the vocabulary (not the rows) leaves only the
//         smaller dh [M, D] to accumulate.
//
// The core: macro tile 256 x 256 of v_mfma_f32_32x32x16_bf16 blocks, as
// 2 x 4 waves with 128 x 64 wave tiles (two waves per SIMD, 128 fp32
// accumulators per lane). Operands go global -> registers -> LDS, 64
// along k per stage, double-buffered in LDS with one barrier per stage: the
// global loads of stage s+1 are in flight while the MFMAs of stage s run,
// and the fragments of k-step kk+1 are read from LDS between the MFMAs of
// k-step kk. LDS rows are padded to 72 elements (144 B), so the 16-byte
// operand reads of consecutive rows fall in distinct banks. Workgroup ids
// are remapped so that the workgroups on one XCD (ids are dealt to the 8
// XCDs in turn) take consecutive tiles, and in the backward products each
// run of 32 of them covers a 4 x 8 block of tiles, sharing A and B tiles in
// that XCD's L2.
#include <type_traits>

#include "vce_kernels.h"

namespace vce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // plain vector: stays in registers

constexpr int LDK = kBK + 8;                         // LDS row stride (elements)
constexpr int WI = 4;                                // 32 x 32 blocks per wave along i
// A workgroup is 2 x NWJ waves; along j a wave holds WJ blocks (in use:
// WJ = 2, NWJ = 4: 512 threads, 256 x 256 macro tile, two waves per SIMD).
template <int WJ, int NWJ> struct Cfg {
    static constexpr int THREADS = 128 * NWJ;
    static constexpr int BJ = 32 * WJ * NWJ;
    static constexpr int RPL = THREADS / 8;                      // tile rows per load instruction
    static constexpr int A_LOADS = kBI * kBK / 8 / THREADS;      // 16-byte loads per thread and stage
    static constexpr int B_LOADS = BJ * kBK / 8 / THREADS;
    static constexpr int STAGE = (kBI + BJ) * LDK;               // elements per stage
    static constexpr size_t LDS = 2 * STAGE * sizeof(uint16_t);
};
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum { EPI_FWD = 0, EPI_GRAD = 1, EPI_STORE = 2 };
// Every product runs 2 x 4 waves with 128 x 64 wave tiles: two waves per
// SIMD hide each other's barrier and load waits (measured faster than 2 x 2
// waves with 256 accumulators per lane for each of the four products).
#define VCE_SHAPE 2, 4

struct GemmArgs {
    const uint16_t *A, *B;
    int64_t lda, ldb;
    int I, J, K;                 // live rows of A and B; K a multiple of kBK
    int n_jtiles;
    // FWD
    int V, tiles_per_split, n_itiles;
    int v_base;                  // GRAD: vocabulary index of A's row 0
    const int32_t *targets;
    float2 *part;
    float *zt;
    // GRAD
    const float *lse, *dloss;
    uint16_t *G, *Gt;
    int64_t ldg, ldgt;
    // STORE
    float *C;
    int64_t ldc;
    int accumulate;
};

__device__ __forceinline__ int xcd_remap(int b, int n) {
    return (n & 7) ? b : (b & 7) * (n >> 3) + (b >> 3);
}

// Tile (ti, tj) of logical workgroup b in an n_i x n_j grid. Each run of 32
// consecutive ids -- the workgroups one XCD holds at a time -- covers a
// 4 x 8 block of tiles, so that they share 4 A tiles and 8 B tiles in that
// XCD's L2 instead of 1 A tile and 32 B tiles.
__device__ __forceinline__ void tile_of(int b, int n_i, int n_j, int &ti, int &tj) {
    if ((n_i & 3) == 0 && (n_j & 7) == 0) {
        const int g = b >> 5, w = b & 31, ngj = n_j >> 3;
        ti = (g / ngj) * 4 + (w >> 3);
        tj = (g % ngj) * 8 + (w & 7);
        return;
    }
    ti = b / n_j;
    tj = b % n_j;
}

__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// (max, sum) pairs in base-2 units: sum_x 2^(x - max).
__device__ __forceinline__ void lse_merge(float &m, float &s, float om, float os) {
    const float mx = fmaxf(m, om);
    if (mx == -INFINITY) return;
    s = s * exp2f(m - mx) + os * exp2f(om - mx);
    m = mx;
}

template <int EPI, int WJ, int NWJ>
__global__ __launch_bounds__(128 * NWJ) void gemm_kernel(GemmArgs p) {   // Cfg::THREADS
    using C = Cfg<WJ, NWJ>;
    constexpr int BJ = C::BJ, A_LOADS = C::A_LOADS, B_LOADS = C::B_LOADS, STAGE = C::STAGE, RPL = C::RPL;
    constexpr int WSJ = 32 * WJ;                     // columns per wave
    extern __shared__ __align__(16) uint16_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wi = wave / NWJ, wj = wave % NWJ;
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    int ti, jt;                    // FWD: ti = vocabulary split; else the row tile of A
    if (EPI == EPI_FWD) {            // measured: the grouping does not help the forward
        ti = b / p.n_jtiles;
        jt = b % p.n_jtiles;
    } else {
        tile_of(b, gridDim.x / p.n_jtiles, p.n_jtiles, ti, jt);
    }
    int it_begin, it_end;
    if (EPI == EPI_FWD) {
        it_begin = ti * p.tiles_per_split;
        it_end = min(it_begin + p.tiles_per_split, p.n_itiles);
    } else {
        it_begin = ti;
        it_end = it_begin + 1;
    }
    const int j0 = jt * BJ;

    // Per-thread global rows of the staged tiles (rows past the live range
    // are clamped to the last live row; their results are never used).
    const int lrow = tid >> 3, lchunk = (tid & 7) * 8;
    const uint16_t *bsrc[B_LOADS];
#pragma unroll
    for (int q = 0; q < B_LOADS; ++q) {
        const int gj = min(j0 + q * RPL + lrow, p.J - 1);
        bsrc[q] = p.B + (int64_t)gj * p.ldb + lchunk;
    }

    // Epilogue state (FWD): per token column of this lane, the running
    // (max, sum) and the target row.
    float run_m[WJ], run_s[WJ];
    int tgt[WJ];
#pragma unroll
    for (int bj = 0; bj < WJ; ++bj) {
        run_m[bj] = -INFINITY;
        run_s[bj] = 0.f;
        tgt[bj] = -1;
        const int m = j0 + wj * WSJ + bj * 32 + (lane & 31);
        if ((EPI == EPI_FWD || EPI == EPI_GRAD) && m < p.J) {
            const int t = p.targets[m];
            tgt[bj] = (t >= 0 && t < p.V) ? t : -1;
        }
    }

    const int nk = p.K / kBK;
    for (int it = it_begin; it < it_end; ++it) {
        const int i0 = it * kBI;
        const uint16_t *asrc[A_LOADS];
#pragma unroll
        for (int q = 0; q < A_LOADS; ++q) {
            const int gi = min(i0 + q * RPL + lrow, p.I - 1);
            asrc[q] = p.A + (int64_t)gi * p.lda + lchunk;
        }
        f32x16 acc[WI][WJ];
#pragma unroll
        for (int bi = 0; bi < WI; ++bi)
#pragma unroll
            for (int bj = 0; bj < WJ; ++bj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.f;

        // Global loads run one stage ahead of the MFMAs (one register set;
        // the accumulators leave no room for a second).
        u32x4 xa[A_LOADS], xb[B_LOADS];
#define VCE_GLOAD(RA, RB, k0)                                                               \
    do {                                                                                    \
        _Pragma("unroll") for (int q = 0; q < A_LOADS; ++q) RA[q] = *(const u32x4 *)(asrc[q] + (k0)); \
        _Pragma("unroll") for (int q = 0; q < B_LOADS; ++q) RB[q] = *(const u32x4 *)(bsrc[q] + (k0)); \
    } while (0)
#define VCE_LSTORE(RA, RB, buf)                                                             \
    do {                                                                                    \
        uint16_t *sa_ = lds + (buf) * STAGE;                                                \
        uint16_t *sb_ = sa_ + kBI * LDK;                                                    \
        _Pragma("unroll") for (int q = 0; q < A_LOADS; ++q)                                 \
            *(u32x4 *)(sa_ + (q * RPL + lrow) * LDK + lchunk) = RA[q];                       \
        _Pragma("unroll") for (int q = 0; q < B_LOADS; ++q)                                 \
            *(u32x4 *)(sb_ + (q * RPL + lrow) * LDK + lchunk) = RB[q];                       \
    } while (0)
#define VCE_FRAGS(F, G, kk)                                                                 \
    do {                                                                                    \
        _Pragma("unroll") for (int bi = 0; bi < WI; ++bi)                                   \
            F[bi] = *(const bf16x8 *)(sa_ + bi * 32 * LDK + (kk) * 16);                     \
        _Pragma("unroll") for (int bj = 0; bj < WJ; ++bj)                                   \
            G[bj] = *(const bf16x8 *)(sb_ + bj * 32 * LDK + (kk) * 16);                     \
    } while (0)
#define VCE_MFMAS(F, G)                                                                     \
    do {                                                                                    \
        _Pragma("unroll") for (int bi = 0; bi < WI; ++bi)                                   \
            _Pragma("unroll") for (int bj = 0; bj < WJ; ++bj)                               \
                acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[bi], G[bj], acc[bi][bj], 0, 0, 0); \
    } while (0)
// One k-step: the MFMAs of (F, G) with the reads of the next fragments
// (FN, GN) spread between them, one read after each of the first MFMAs.
#define VCE_STEP(F, G, FN, GN, kkn)                                                          \
    do {                                                                                    \
        VCE_FRAGS(FN, GN, kkn);                                                             \
        VCE_MFMAS(F, G);                                                                    \
        _Pragma("unroll") for (int q_ = 0; q_ < WI + WJ; ++q_) {                            \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                              \
        }                                                                                   \
        __builtin_amdgcn_sched_group_barrier(0x008, WI * WJ - WI - WJ, 0);                  \
        __builtin_amdgcn_sched_barrier(0);                                                  \
    } while (0)
// The fragments of k-step kk+1 are read while the MFMAs of k-step kk run;
// the scheduling barriers keep the compiler from hoisting every read of
// the stage (which would need 96 more registers).
#define VCE_COMPUTE(buf)                                                                    \
    do {                                                                                    \
        const uint16_t *sa_ = lds + (buf) * STAGE + (wi * 128 + (lane & 31)) * LDK + (lane >> 5) * 8; \
        const uint16_t *sb_ = lds + (buf) * STAGE + kBI * LDK + (wj * WSJ + (lane & 31)) * LDK + (lane >> 5) * 8; \
        bf16x8 f0[WI], g0[WJ], f1[WI], g1[WJ];                                              \
        VCE_FRAGS(f0, g0, 0);                                                               \
        __builtin_amdgcn_sched_barrier(0);                                                  \
        VCE_STEP(f0, g0, f1, g1, 1);                                                        \
        VCE_STEP(f1, g1, f0, g0, 2);                                                        \
        VCE_STEP(f0, g0, f1, g1, 3);                                                        \
        VCE_MFMAS(f1, g1);                                                                  \
    } while (0)

        __syncthreads();               // the previous tile's epilogue may still read LDS
        VCE_GLOAD(xa, xb, 0);
        VCE_LSTORE(xa, xb, 0);
        __syncthreads();
        for (int s = 0; s < nk; ++s) {
            const int buf = s & 1;
            if (s + 1 < nk) VCE_GLOAD(xa, xb, (s + 1) * kBK);
            VCE_COMPUTE(buf);
            if (s + 1 < nk) VCE_LSTORE(xa, xb, buf ^ 1);
            __syncthreads();
        }

        // Accumulator (bi, bj, r) of lane l is C[i][j] with
        //   i = i0 + wi*128 + bi*32 + 8*(r/4) + 4*(l/32) + r%4,
        //   j = j0 + wj*32*WJ + bj*32 + l%32.
        const int ib = i0 + wi * 128 + 4 * (lane >> 5);
        // tiles wholly inside the row range skip the per-element bounds tests
        const bool inside = i0 + 2 * 128 <= (EPI == EPI_FWD ? p.V : p.I);
        if (EPI == EPI_FWD) {
            // (max, sum) of this lane's column over the tile's rows, folded
            // into the running pair; exp2 of arguments <= 0 on the hardware
            // instruction (v_exp_f32)
            auto fold = [&](int bj, auto IN) {
                constexpr bool in = decltype(IN)::value;
                float tmax = -INFINITY;
#pragma unroll
                for (int bi = 0; bi < WI; ++bi)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int v = ib + bi * 32 + 8 * (r >> 2) + (r & 3);
                        if (in || v < p.V) tmax = fmaxf(tmax, acc[bi][bj][r]);
                    }
                tmax *= kLog2e;
                const float mnew = fmaxf(run_m[bj], tmax);
                if (mnew != -INFINITY) {
                    float sum = 0.f;
#pragma unroll
                    for (int bi = 0; bi < WI; ++bi)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int v = ib + bi * 32 + 8 * (r >> 2) + (r & 3);
                            const float e = __builtin_amdgcn_exp2f(fmaf(acc[bi][bj][r], kLog2e, -mnew));
                            sum += (in || v < p.V) ? e : 0.f;
                        }
                    run_s[bj] = run_s[bj] * __builtin_amdgcn_exp2f(run_m[bj] - mnew) + sum;
                    run_m[bj] = mnew;
                }
            };
#pragma unroll
            for (int bj = 0; bj < WJ; ++bj) {
                if (inside) fold(bj, std::true_type{});
                else fold(bj, std::false_type{});
                // Target logit: the one lane that holds row t of this column.
                const int d = tgt[bj] - ib;
                if (d >= 0 && d < 128 && ((d >> 2) & 1) == 0) {
                    const int tbi = d >> 5, tr = ((d >> 3) & 3) * 4 + (d & 3);
                    float z = 0.f;
#pragma unroll
                    for (int bi = 0; bi < WI; ++bi)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (bi == tbi && r == tr) z = acc[bi][bj][r];
                    p.zt[j0 + wj * WSJ + bj * 32 + (lane & 31)] = z;
                }
            }
        } else if (EPI == EPI_GRAD) {
            // G^T [v][m]: neighbouring lanes hold neighbouring m, so an even
            // lane stores (m, m+1) of one row and its odd neighbour (m-1, m)
            // of the next, after one lane exchange: 4-byte stores.
            // G [m][v]: a lane holds 4 consecutive v of one m; they go to LDS
            // as the tile [m][v] and leave as 16-byte row segments (a direct
            // store would touch a different row in every lane).
            constexpr int TLD = kBI + 8;                 // LDS row stride of the [m][v] tile
            const bool odd = lane & 1;
#pragma unroll
            for (int bj = 0; bj < WJ; ++bj) {
                const int ml = wj * WSJ + bj * 32 + (lane & 31);
                const int m = j0 + ml;
                const bool live = m < p.J && tgt[bj] >= 0;
                const float l2 = live ? p.lse[m] * kLog2e : 0.f;
                const float dl = live ? p.dloss[m] : 0.f;
                const int tl = tgt[bj] - p.v_base;       // target as a local row
                uint16_t *trow = lds + ml * TLD + wi * 128 + 4 * (lane >> 5);
                uint16_t *gtcol = p.Gt + (m & ~1);
#pragma unroll
                for (int bi = 0; bi < WI; ++bi) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int vb = ib + bi * 32 + 8 * r4;
                        uint32_t g[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int v = vb + e;
                            float x = __builtin_amdgcn_exp2f(fmaf(acc[bi][bj][r4 * 4 + e], kLog2e, -l2));
                            x = (v == tl) ? x - 1.f : x;
                            x = (live && (inside || v < p.I)) ? x * dl : 0.f;
                            g[e] = to_bf16(x);
                        }
                        uint2 pk;
                        pk.x = g[0] | (g[1] << 16);
                        pk.y = g[2] | (g[3] << 16);
                        *(uint2 *)(trow + bi * 32 + 8 * r4) = pk;
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const uint32_t recv = __shfl_xor(odd ? g[2 * q] : g[2 * q + 1], 1);
                            const uint32_t word = odd ? (recv | (g[2 * q + 1] << 16)) : (g[2 * q] | (recv << 16));
                            *(uint32_t *)(gtcol + (int64_t)(vb + 2 * q + (odd ? 1 : 0)) * p.ldgt) = word;
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
            constexpr int CPR = kBI / 8;                 // 16-byte segments per row
#pragma unroll 4
            for (int c = tid; c < BJ * CPR; c += C::THREADS) {
                const int row = c / CPR, seg = c % CPR;
                const u32x4 val = *(const u32x4 *)(lds + row * TLD + seg * 8);
                *(u32x4 *)(p.G + (int64_t)(j0 + row) * p.ldg + i0 + seg * 8) = val;
            }
        } else {
#pragma unroll
            for (int bj = 0; bj < WJ; ++bj) {
                const int j = j0 + wj * WSJ + bj * 32 + (lane & 31);
                if (j >= p.J) continue;
#pragma unroll
                for (int bi = 0; bi < WI; ++bi)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = ib + bi * 32 + 8 * (r >> 2) + (r & 3);
                        if (i < p.I) {
                            float *c = p.C + (int64_t)i * p.ldc + j;
                            *c = p.accumulate ? *c + acc[bi][bj][r] : acc[bi][bj][r];
                        }
                    }
            }
        }
    }

#undef VCE_GLOAD
#undef VCE_LSTORE
#undef VCE_COMPUTE
#undef VCE_STEP
#undef VCE_FRAGS
#undef VCE_MFMAS

    if (EPI == EPI_FWD) {
        // Merge the two lanes that share each column, then the two waves
        // (wi = 0, 1) that share it, and write this split's partial.
#pragma unroll
        for (int bj = 0; bj < WJ; ++bj) {
            const float om = __shfl_xor(run_m[bj], 32), os = __shfl_xor(run_s[bj], 32);
            lse_merge(run_m[bj], run_s[bj], om, os);
        }
        float2 *red = (float2 *)lds;
        __syncthreads();
        if (wi == 1 && lane < 32)
#pragma unroll
            for (int bj = 0; bj < WJ; ++bj) red[wj * WSJ + bj * 32 + lane] = make_float2(run_m[bj], run_s[bj]);
        __syncthreads();
        if (wi == 0 && lane < 32) {
            const int split = ti;
#pragma unroll
            for (int bj = 0; bj < WJ; ++bj) {
                const float2 o = red[wj * WSJ + bj * 32 + lane];
                lse_merge(run_m[bj], run_s[bj], o.x, o.y);
                const int m = j0 + wj * WSJ + bj * 32 + lane;
                if (m < p.J) p.part[(int64_t)split * p.J + m] = make_float2(run_m[bj], run_s[bj]);
            }
        }
    }
}

// lse and loss per row from the splits' partials.
__global__ __launch_bounds__(256) void combine_kernel(int M, int V, int nsplit, const float2 *part,
                                                      const float *zt, const int32_t *targets,
                                                      float *loss, float *lse) {
    const int m = blockIdx.x * 256 + threadIdx.x;
    if (m >= M) return;
    float mx = -INFINITY, s = 0.f;
    for (int q = 0; q < nsplit; ++q) {
        const float2 o = part[(int64_t)q * M + m];
        lse_merge(mx, s, o.x, o.y);
    }
    const float l = (mx + log2f(s)) * kLn2;
    lse[m] = l;
    const int t = targets[m];
    loss[m] = (t >= 0 && t < V) ? l - zt[m] : 0.f;
}

// out[c][r] = in[r][c] for r < R, c < C, and 0 for R <= r < ldo: a 64 x 64
// tile per workgroup through LDS (ldo a multiple of 64).
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t *in, int64_t ldi, int R, int C,
                                                            uint16_t *out, int64_t ldo) {
    __shared__ uint16_t t[64][66];
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int r = r0 + q * 4 + ty, c = c0 + tx;
        t[q * 4 + ty][tx] = (r < R && c < C) ? in[(int64_t)r * ldi + c] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int c = c0 + q * 4 + ty, r = r0 + tx;
        if (c < C) out[(int64_t)c * ldo + r] = t[tx][q * 4 + ty];
    }
}

template <int EPI, int WJ, int NWJ>
hipError_t launch_gemm(const GemmArgs &a, int blocks, hipStream_t stream) {
    using C = Cfg<WJ, NWJ>;
    hipError_t e = hipFuncSetAttribute((const void *)gemm_kernel<EPI, WJ, NWJ>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_kernel<EPI, WJ, NWJ>), dim3((unsigned)blocks), dim3(C::THREADS), C::LDS, stream, a);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t *in, int64_t ldi, int R, int C, uint16_t *out, int64_t ldo,
                            hipStream_t stream) {
    dim3 grid((unsigned)(ldo / 64), (unsigned)((C + 63) / 64));
    hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(256), 0, stream, in, ldi, R, C, out, ldo);
    return hipGetLastError();
}

}  // namespace

FwdPlan fwd_plan(int M, int V) {
    FwdPlan f;
    f.n_itiles = (int)((V + kBI - 1) / kBI);
    f.n_jtiles = (int)((M + kBJ - 1) / kBJ);
    const int want = (2048 + f.n_jtiles - 1) / f.n_jtiles;
    const int ns = want < f.n_itiles ? want : f.n_itiles;
    f.tiles_per_split = (f.n_itiles + ns - 1) / ns;
    f.nsplit = (f.n_itiles + f.tiles_per_split - 1) / f.tiles_per_split;
    return f;
}

hipError_t launch_forward(const FwdArgs &a, hipStream_t stream) {
    const FwdPlan f = fwd_plan(a.M, a.V);
    GemmArgs g{};
    g.A = a.w; g.lda = a.D; g.I = a.V;
    g.B = a.h; g.ldb = a.D; g.J = a.M;
    g.K = a.D;
    g.n_jtiles = f.n_jtiles;
    g.V = a.V; g.tiles_per_split = f.tiles_per_split; g.n_itiles = f.n_itiles;
    g.targets = a.targets; g.part = a.part; g.zt = a.zt;
    hipError_t e = launch_gemm<EPI_FWD, VCE_SHAPE>(g, f.n_jtiles * f.nsplit, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((a.M + 255) / 256)), dim3(256), 0, stream, a.M, a.V,
                       f.nsplit, a.part, a.zt, a.targets, a.loss, a.lse);
    return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs &a, hipStream_t stream) {
    hipError_t e;
    const int64_t Vp = round_up(a.V, kBI);
    const int64_t Mp = round_up(a.M, kBJ);
    const int64_t Vcp = round_up(a.Vc, kBI);
    if ((e = launch_transpose(a.w, a.D, a.V, a.D, a.wt, Vp, stream)) != hipSuccess) return e;
    if ((e = launch_transpose(a.h, a.D, a.M, a.D, a.ht, Mp, stream)) != hipSuccess) return e;
    for (int v0 = 0; v0 < a.V; v0 += a.Vc) {
        const int vc = a.V - v0 < a.Vc ? a.V - v0 : a.Vc;
        const int vcp = (int)round_up(vc, kBI);

        GemmArgs g{};                 // G and G^T for vocabulary rows [v0, v0 + vc)
        g.A = a.w + (int64_t)v0 * a.D; g.lda = a.D; g.I = vc;
        g.B = a.h; g.ldb = a.D; g.J = a.M;
        g.K = a.D; g.V = a.V; g.v_base = v0;
        g.n_jtiles = (int)(Mp / kBJ);
        g.targets = a.targets; g.lse = a.lse; g.dloss = a.dloss;
        g.G = a.g; g.ldg = Vcp; g.Gt = a.gt; g.ldgt = Mp;
        if ((e = launch_gemm<EPI_GRAD, VCE_SHAPE>(g, vcp / kBI * g.n_jtiles, stream)) != hipSuccess) return e;

        GemmArgs d{};                 // dh (+)= G W over the chunk's vocabulary rows
        d.A = a.g; d.lda = Vcp; d.I = a.M;
        d.B = a.wt + v0; d.ldb = Vp; d.J = a.D;
        d.K = vcp;
        d.n_jtiles = (a.D + Cfg<VCE_SHAPE>::BJ - 1) / Cfg<VCE_SHAPE>::BJ;
        d.C = a.dh; d.ldc = a.D; d.accumulate = v0 > 0;
        if ((e = launch_gemm<EPI_STORE, VCE_SHAPE>(d, (int)(Mp / kBI) * d.n_jtiles, stream)) != hipSuccess) return e;

        GemmArgs w{};                 // dW rows [v0, v0 + vc) = G^T h
        w.A = a.gt; w.lda = Mp; w.I = vc;
        w.B = a.ht; w.ldb = Mp; w.J = a.D;
        w.K = (int)Mp;
        w.n_jtiles = (a.D + Cfg<VCE_SHAPE>::BJ - 1) / Cfg<VCE_SHAPE>::BJ;
        w.C = a.dw + (int64_t)v0 * a.D; w.ldc = a.D; w.accumulate = 0;
        if ((e = launch_gemm<EPI_STORE, VCE_SHAPE>(w, vcp / kBI * w.n_jtiles, stream)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace vce
