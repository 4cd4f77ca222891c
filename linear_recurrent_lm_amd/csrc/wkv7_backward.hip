// WKV-7 backward from 16-token state checkpoints, token order.
//
// Reverse-mode of S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T + v_t k_t^T,
// y_t = S_t r_t for L = sum <dy, y> + <ds_out, S_T>. With G = dL/dS_t and
// sa_t = S_{t-1} a_t, each token (last to first) does
//     G      += dy_t r_t^T
//     dr_t    = S_t^T dy_t          dv_t = G k_t        dsa = G b_t
//     dk_t    = G^T v_t             db_t = G^T sa_t
//     dw_t[j] = sum_i G[i,j] S_{t-1}[i,j]               da_t = S_{t-1}^T dsa
//     G       = G diag(w_t) + dsa a_t^T
// The states S_{t-1} of a chunk are recomputed forward from its checkpoint
// (the state entering the chunk), never reconstructed by dividing by w, as
// the rwkv-metal page's section "The Metal WKV-7 kernel" motivates.
//
// One 1024-thread workgroup per (sequence, head). Thread tid owns row
// i = tid/16 and columns 4*(tid%16) .. +3 of G and of the recomputed states,
// which stay in registers for the whole chunk. Row sums (sa, dv, dsa) reduce
// over the 16 lanes of a row; column sums (dr, dk, db, dw, da) reduce over the
// 4 rows inside a wave by lane exchange and over the 16 waves through LDS.
#include "wkv7_kernels.h"

namespace wkv7 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
enum { SR = 0, SW, SK, SA, SB, SV, SDY, NSTREAM };

__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 8, 16);
    return x;
}

__device__ __forceinline__ float sum_rows_in_wave(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

template <typename TI>
__global__ __launch_bounds__(kThreads) void bwd_token_kernel(BwdArgs p) {
    const int H = p.seg.H;
    const int unit = blockIdx.x;
    const int h = unit % H;
    const int s = unit / H;
    const Unit u = resolve_unit(p.seg, s);
    const int tid = threadIdx.x;
    const int i = tid >> 4;
    const int j0 = (tid & 15) * 4;
    const int wave = tid >> 6;
    const bool row_leader = (tid & 15) == 0;
    const bool wave_row0 = ((tid >> 4) & 3) == 0;

    __shared__ float tin[kChunk][NSTREAM][kN];
    __shared__ float red[2][kWaves][5][kN];

    TI *__restrict__ dvp = (TI *)p.dv;

    const int64_t sidx = ((int64_t)s * H + h) * (kN * kN) + (int64_t)i * kN + j0;
    float G[4];
    if (p.ds_out) {
        const float4 q = *(const float4 *)(p.ds_out + sidx);
        G[0] = q.x; G[1] = q.y; G[2] = q.z; G[3] = q.w;
    } else {
        G[0] = G[1] = G[2] = G[3] = 0.f;
    }

    const int64_t ts = (int64_t)H * kN;
    const int64_t base = (u.start * H + h) * kN;
    const int nchunks = (u.len + kChunk - 1) / kChunk;

#pragma unroll 1
    for (int c = nchunks - 1; c >= 0; --c) {
        const int t0 = c * kChunk;
        const int L = min(kChunk, u.len - t0);
        __syncthreads();
        for (int idx = tid; idx < L * NSTREAM * kN; idx += kThreads) {
            const int t = idx / (NSTREAM * kN);
            const int rem = idx - t * (NSTREAM * kN);
            const int st = rem / kN;
            const int e = rem - st * kN;
            const int64_t o = base + (int64_t)(t0 + t) * ts + e;
            const void *src = st == SR ? p.r : st == SW ? p.w : st == SK ? p.k
                            : st == SA ? p.a : st == SB ? p.b : st == SV ? p.v : p.dy;
            tin[t][st][e] = src ? IO<TI>::ld((const TI *)src, o) : 0.f;
        }
        float hist[kChunk + 1][4];
        {
            const float4 q = *(const float4 *)(p.ckpt + ((u.ckpt + c) * H + h) * (int64_t)(kN * kN) +
                                               (int64_t)i * kN + j0);
            hist[0][0] = q.x; hist[0][1] = q.y; hist[0][2] = q.z; hist[0][3] = q.w;
        }
        __syncthreads();

        float sa_r[kChunk];
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
            if (t < L) {
                float part = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) part = fmaf(hist[t][e], tin[t][SA][j0 + e], part);
                const float sa = sum16(part);
                sa_r[t] = sa;
                const float vi = tin[t][SV][i];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hist[t + 1][e] = fmaf(hist[t][e], tin[t][SW][j0 + e],
                                          fmaf(sa, tin[t][SB][j0 + e], vi * tin[t][SK][j0 + e]));
            }
        }

#pragma unroll
        for (int t = kChunk - 1; t >= 0; --t) {
            if (t < L) {
                const float dyi = tin[t][SDY][i];
                const float vi = tin[t][SV][i];
                const float sa = sa_r[t];
                float rr[4], ww[4], kk[4], aa[4], bb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rr[e] = tin[t][SR][j0 + e]; ww[e] = tin[t][SW][j0 + e];
                    kk[e] = tin[t][SK][j0 + e]; aa[e] = tin[t][SA][j0 + e];
                    bb[e] = tin[t][SB][j0 + e];
                }
                float part[5][4];
                float dvq = 0.f, dsq = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    G[e] = fmaf(dyi, rr[e], G[e]);
                    part[0][e] = hist[t + 1][e] * dyi;
                    dvq = fmaf(G[e], kk[e], dvq);
                    dsq = fmaf(G[e], bb[e], dsq);
                }
                const float dv = sum16(dvq);
                const float dsa = sum16(dsq);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    part[1][e] = G[e] * vi;
                    part[2][e] = G[e] * sa;
                    part[3][e] = G[e] * hist[t][e];
                    part[4][e] = dsa * hist[t][e];
                    G[e] = fmaf(G[e], ww[e], dsa * aa[e]);
                }
#pragma unroll
                for (int g = 0; g < 5; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) part[g][e] = sum_rows_in_wave(part[g][e]);
                if (wave_row0) {
#pragma unroll
                    for (int g = 0; g < 5; ++g)
#pragma unroll
                        for (int e = 0; e < 4; ++e) red[t & 1][wave][g][j0 + e] = part[g][e];
                }
                const int64_t ot = base + (int64_t)(t0 + t) * ts;
                if (row_leader) IO<TI>::st(dvp, ot + i, dv);
                __syncthreads();
                if (tid < 5 * kN) {
                    const int g = tid >> 6, col = tid & 63;
                    float acc = 0.f;
#pragma unroll
                    for (int q = 0; q < kWaves; ++q) acc += red[t & 1][q][g][col];
                    void *dst = g == 0 ? p.dr : g == 1 ? p.dk : g == 2 ? p.db : g == 3 ? p.dw : p.da;
                    IO<TI>::st((TI *)dst, ot + col, acc);
                }
            }
        }
    }
    if (p.ds0) *(float4 *)(p.ds0 + sidx) = make_float4(G[0], G[1], G[2], G[3]);
}

}  // namespace

hipError_t launch_backward(const BwdArgs &a, hipStream_t stream) {
    const int S = a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B;
    const dim3 grid((unsigned)((int64_t)S * a.seg.H));
    if (a.dtype == 1)
        hipLaunchKernelGGL(bwd_token_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(bwd_token_kernel<float>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace wkv7
