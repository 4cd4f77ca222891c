// WKV-7 backward at head size 128, token by token, from the 16-token state
// checkpoints of the forward. Reverse-mode through
//     S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T + v_t k_t^T,   y_t = S_t r_t
// with dS the gradient of the state after token t (ds_out after the last):
//     dS += dy_t r_t^T;                 dr_t = S_t^T dy_t
//     dv_t = dS k_t;   dk_t = dS^T v_t;  dsa = dS b_t;   db_t = dS^T sa_t
//     dw_t = colsum(dS o S_{t-1});       da_t = S_{t-1}^T dsa
//     dS <- dS diag(w_t) + dsa a_t^T    (the gradient of the state before t)
// where sa_t = S_{t-1} a_t. S_{t-1} is never rebuilt from S_t (that divides by
// w): each chunk's states are recomputed forward from its checkpoint.
//
// The value rows of the state evolve independently, in the recurrence and in
// its adjoint: dS's row i needs only row i of S, v_i and dy_i. A workgroup
// therefore owns 8 value rows of one (sequence, head) through the whole
// sequence, in reverse: 16 workgroups per unit. Thread t holds keys 4 (t % 32)
// .. + 3 of row t / 32 (a wave holds two rows), with dS and, for one half of
// a chunk at a time, the 8 recomputed states of its 4 elements and sa in
// registers. Row sums (S a,
// dS k, dS b) reduce over the 32 lanes of a row. The key-indexed gradients
// (dr, dk, db, dw, da) are sums over all 128 rows: each workgroup adds its
// 8 rows' share to fp32 accumulators in the workspace with hardware atomics,
// and a last kernel writes them out in the gradients' dtype; dv and ds0 are
// per row and written directly.
//
// Per chunk the r, w, k, a, b rows of its 16 tokens and the block's v and dy
// are staged in LDS as fp32 (w exponentiated for log-decay input), from
// registers loaded while the previous chunk ran.
#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr int kWN = 128;            // head size
constexpr int kRowsPerBlock = 8;
constexpr int kBlocksPerUnit = kWN / kRowsPerBlock;
constexpr int kWThreads = 256;
enum { SW = 0, SA, SB, SK, SR, NSTAGE };     // staged key-indexed rows
enum { GR = 0, GK, GB, GW, GA, NACC };       // accumulated key-indexed gradients

// LDS (floats): staged rows [NSTAGE][16][128], v and dy of the block's rows
// [2][16][8], partial column sums [8 rows][NACC][128]: 62.5 KB, two
// workgroups per CU
constexpr int L_ST = 0;
constexpr int L_VD = L_ST + NSTAGE * kChunk * kWN;
constexpr int L_PART = L_VD + 2 * kChunk * kRowsPerBlock;
constexpr int L_TOTAL = L_PART + kRowsPerBlock * NACC * kWN;

// 8 consecutive elements in flight (one 16-byte load, two for fp32)
template <typename TI> struct Raw8;
template <> struct Raw8<uint16_t> { uint4 q; };
template <> struct Raw8<_Float16> { uint4 q; };
template <> struct Raw8<float> { float4 q[2]; };
__device__ __forceinline__ void ld8(const uint16_t *p, Raw8<uint16_t> &r) { r.q = *(const uint4 *)p; }
__device__ __forceinline__ void ld8(const _Float16 *p, Raw8<_Float16> &r) { r.q = *(const uint4 *)p; }
__device__ __forceinline__ void ld8(const float *p, Raw8<float> &r) {
    r.q[0] = *(const float4 *)p;
    r.q[1] = *(const float4 *)(p + 4);
}
__device__ __forceinline__ void un8(const Raw8<uint16_t> &r, float *x) {
    const uint32_t u[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(u[e] << 16);
        x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
}
__device__ __forceinline__ void un8(const Raw8<_Float16> &r, float *x) {
    const uint32_t u[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = half_lo(u[e]);
        x[2 * e + 1] = half_hi(u[e]);
    }
}
__device__ __forceinline__ void un8(const Raw8<float> &r, float *x) {
    x[0] = r.q[0].x; x[1] = r.q[0].y; x[2] = r.q[0].z; x[3] = r.q[0].w;
    x[4] = r.q[1].x; x[5] = r.q[1].y; x[6] = r.q[1].z; x[7] = r.q[1].w;
}

// sum over the 32 lanes of a row (lanes 0-31 or 32-63 of the wave)
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) x += __shfl_xor(x, m, 32);
    return x;
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kWThreads, 2) void bwd128_kernel(BwdArgs p, float *acc, int32_t units) {
    __shared__ __align__(16) float sm[L_TOTAL];
    const int g8 = blockIdx.x / (8 * kBlocksPerUnit), wq = blockIdx.x % (8 * kBlocksPerUnit);
    const int unit = g8 * 8 + (wq & 7);             // a unit's row blocks share an XCD
    const int rb = wq >> 3;
    if (unit >= units) return;
    const int H = p.seg.H;
    const int h = unit % H, sq = unit / H;
    const Unit u = resolve_unit(p.seg, sq);
    const int tid = threadIdx.x;
    const int r8 = tid >> 5, kq = tid & 31;
    const int row = rb * kRowsPerBlock + r8;        // value row of this thread
    const int64_t ts = (int64_t)H * kWN;            // token pitch of a stream
    const int64_t base = (u.start * H + h) * kWN;
    const int64_t sbase = ((int64_t)sq * H + h) * (int64_t)(kWN * kWN);
    const int64_t toks = (int64_t)p.seg.B * p.seg.T;
    const int nch = (u.len + kChunk - 1) / kChunk;

    // dS: row `row`, keys 4 kq .. 4 kq + 3
    float4 dS = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.ds_out) dS = *(const float4 *)(p.ds_out + sbase + (int64_t)row * kWN + 4 * kq);

    // staging: thread t loads 8 keys (t % 16) * 8 of token t / 16 of each row
    // stream, and (t < 128) v or dy of row t % 8 of token (t / 8) % 16
    const int se = tid >> 4, sc = (tid & 15) * 8;
    const TI *srcs[NSTAGE] = {(const TI *)p.w, (const TI *)p.a, (const TI *)p.b,
                              (const TI *)p.k, (const TI *)p.r};
    Raw8<TI> raw[NSTAGE];
    TI rvd = TI(0);
    const int ve = (tid >> 3) & 15, vr = tid & 7;
    const bool vd_dy = tid >= 128 && tid < 256;
    auto issue = [&](int cc) {
        const int Lc = min(kChunk, u.len - cc * kChunk);
        const int64_t t0 = (int64_t)cc * kChunk;
        const int64_t o = base + (t0 + min(se, Lc - 1)) * ts + sc;
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s) ld8(srcs[s] + o, raw[s]);
        const int64_t ov = base + (t0 + min(ve, Lc - 1)) * ts + rb * kRowsPerBlock + vr;
        if (!vd_dy) rvd = ((const TI *)p.v)[ov];
        else rvd = p.dy ? ((const TI *)p.dy)[ov] : TI(0);
    };
    auto stage = [&]() {
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s) {
            float x[8];
            un8(raw[s], x);
            if (s == SW) decay_of<8>(x, p.logw);
            float *d = sm + L_ST + (s * kChunk + se) * kWN + sc;
            *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
            *(float4 *)(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
        }
        sm[L_VD + (vd_dy ? kChunk * kRowsPerBlock : 0) + ve * kRowsPerBlock + vr] = IO<TI>::ld(&rvd, 0);
    };
    auto rowv = [&](int s, int e) { return *(const float4 *)(sm + L_ST + (s * kChunk + e) * kWN + 4 * kq); };

    if (nch > 0) issue(nch - 1);
#pragma unroll 1
    for (int c = nch - 1; c >= 0; --c) {
        const int Lc = min(kChunk, u.len - c * kChunk);
        const int64_t t0 = (int64_t)c * kChunk;
        __syncthreads();                            // the previous chunk is done with the staged rows
        stage();
        if (c > 0) issue(c - 1);
        const float4 S0 = *(const float4 *)(p.ckpt + ((u.ckpt + c) * H + h) * (int64_t)(kWN * kWN) +
                                            (int64_t)row * kWN + 4 * kq);
        __syncthreads();
        // one forward step of this thread's 4 elements; returns sa = S a
        auto step = [&](float4 &S, int e) {
            const float4 w4 = rowv(SW, e), a4 = rowv(SA, e), b4 = rowv(SB, e), k4 = rowv(SK, e);
            const float vi = sm[L_VD + e * kRowsPerBlock + r8];
            const float s_ = row_sum(S.x * a4.x + S.y * a4.y + S.z * a4.z + S.w * a4.w);
            S.x = fmaf(S.x, w4.x, fmaf(s_, b4.x, vi * k4.x));
            S.y = fmaf(S.y, w4.y, fmaf(s_, b4.y, vi * k4.y));
            S.z = fmaf(S.z, w4.z, fmaf(s_, b4.z, vi * k4.z));
            S.w = fmaf(S.w, w4.w, fmaf(s_, b4.w, vi * k4.w));
            return s_;
        };
        // the chunk in two halves of 8 tokens, the later one first: the
        // states before each token of a half are recomputed from the
        // checkpoint (the later half's start from the first half's end)
#pragma unroll 1
        for (int half = 1; half >= 0; --half) {
            const int e0 = 8 * half;
            if (e0 >= Lc) continue;
            float4 S = S0;
            if (half == 1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) step(S, e);
            }
            float4 Sp[8];
            float sa[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Sp[e] = S;
                sa[e] = 0.f;
                if (e0 + e < Lc) sa[e] = step(S, e0 + e);
            }
#pragma unroll
            for (int e = 7; e >= 0; --e) {
                const int te = e0 + e;
                if (te < Lc) {
                    const float4 w4 = rowv(SW, te), a4 = rowv(SA, te), b4 = rowv(SB, te);
                    const float4 k4 = rowv(SK, te), r4 = rowv(SR, te);
                    const float vi = sm[L_VD + te * kRowsPerBlock + r8];
                    const float dyi = sm[L_VD + (kChunk + te) * kRowsPerBlock + r8];
                    const float4 P = Sp[e];
                    const float s_ = sa[e];
                    float4 St;                                  // S_t
                    St.x = fmaf(P.x, w4.x, fmaf(s_, b4.x, vi * k4.x));
                    St.y = fmaf(P.y, w4.y, fmaf(s_, b4.y, vi * k4.y));
                    St.z = fmaf(P.z, w4.z, fmaf(s_, b4.z, vi * k4.z));
                    St.w = fmaf(P.w, w4.w, fmaf(s_, b4.w, vi * k4.w));
                    dS.x = fmaf(dyi, r4.x, dS.x);
                    dS.y = fmaf(dyi, r4.y, dS.y);
                    dS.z = fmaf(dyi, r4.z, dS.z);
                    dS.w = fmaf(dyi, r4.w, dS.w);
                    const float dvi = row_sum(dS.x * k4.x + dS.y * k4.y + dS.z * k4.z + dS.w * k4.w);
                    const float dsa = row_sum(dS.x * b4.x + dS.y * b4.y + dS.z * b4.z + dS.w * b4.w);
                    if (kq == 0) IO<TO>::st((TO *)p.dv, base + (t0 + te) * ts + row, dvi);
                    // this row's share of the key-indexed gradients
                    float *pt = sm + L_PART + r8 * NACC * kWN + 4 * kq;
                    *(float4 *)(pt + GR * kWN) = make_float4(St.x * dyi, St.y * dyi, St.z * dyi, St.w * dyi);
                    *(float4 *)(pt + GK * kWN) = make_float4(dS.x * vi, dS.y * vi, dS.z * vi, dS.w * vi);
                    *(float4 *)(pt + GB * kWN) = make_float4(dS.x * s_, dS.y * s_, dS.z * s_, dS.w * s_);
                    *(float4 *)(pt + GW * kWN) = make_float4(dS.x * P.x, dS.y * P.y, dS.z * P.z, dS.w * P.w);
                    *(float4 *)(pt + GA * kWN) = make_float4(P.x * dsa, P.y * dsa, P.z * dsa, P.w * dsa);
                    dS.x = fmaf(dS.x, w4.x, dsa * a4.x);
                    dS.y = fmaf(dS.y, w4.y, dsa * a4.y);
                    dS.z = fmaf(dS.z, w4.z, dsa * a4.z);
                    dS.w = fmaf(dS.w, w4.w, dsa * a4.w);
                    __syncthreads();
                    // the block's 8 rows summed, then added across the unit's blocks
                    if (tid < kWN) {
                        const float *q = sm + L_PART + tid;
                        const int64_t o = ((t0 + te + u.start) * H + h) * kWN + tid;
#pragma unroll
                        for (int g = 0; g < NACC; ++g) {
                            float x = 0.f;
#pragma unroll
                            for (int r = 0; r < kRowsPerBlock; ++r) x += q[(r * NACC + g) * kWN];
                            if (g == GW && p.logw) x *= sm[L_ST + (SW * kChunk + te) * kWN + tid];
                            unsafeAtomicAdd(acc + (int64_t)g * toks * ts + o, x);
                        }
                    }
                    __syncthreads();                    // the partials are free for the next token
                }
            }
        }
    }
    if (p.ds0) *(float4 *)(p.ds0 + sbase + (int64_t)row * kWN + 4 * kq) = dS;
}

__global__ void bwd128_zero_kernel(float4 *p, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// accumulators -> dr, dk, db, dw, da in the gradients' dtype
template <typename TO>
__global__ void bwd128_finish_kernel(BwdArgs p, const float *acc, int64_t n) {
    void *outs[NACC] = {p.dr, p.dk, p.db, p.dw, p.da};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
#pragma unroll
        for (int g = 0; g < NACC; ++g) IO<TO>::st((TO *)outs[g], i, acc[(int64_t)g * n + i]);
    }
}

template <typename TI, typename TO>
hipError_t launch_t(const BwdArgs &a, float *acc, hipStream_t stream) {
    const int64_t units = (int64_t)(a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B) * a.seg.H;
    const int64_t n = (int64_t)a.seg.B * a.seg.T * a.seg.H * kWN;
    hipLaunchKernelGGL(bwd128_zero_kernel, dim3(2048), dim3(256), 0, stream, (float4 *)acc, (int64_t)NACC * n / 4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t blocks = (units + 7) / 8 * 8 * kBlocksPerUnit;
    hipLaunchKernelGGL((bwd128_kernel<TI, TO>), dim3((unsigned)blocks), dim3(kWThreads), 0, stream, a, acc,
                       (int32_t)units);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd128_finish_kernel<TO>, dim3(2048), dim3(256), 0, stream, a, (const float *)acc, n);
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_ti(const BwdArgs &a, float *acc, hipStream_t stream) {
    if (a.grad_f32) return launch_t<TI, float>(a, acc, stream);
    return launch_t<TI, TI>(a, acc, stream);
}

}  // namespace

hipError_t launch_backward128(const BwdArgs &a, float *acc, hipStream_t stream) {
    if (a.dtype == 1) return launch_ti<uint16_t>(a, acc, stream);
    if (a.dtype == 2) return launch_ti<_Float16>(a, acc, stream);
    return launch_ti<float>(a, acc, stream);
}

}  // namespace wkv7
