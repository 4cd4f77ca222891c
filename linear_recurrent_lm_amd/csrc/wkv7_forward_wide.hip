// WKV-7 forward at head size 128 (the matched head size of the rwkv-lab
// page's GDN conversion target), token by token:
//     S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T + v_t k_t^T,   y_t = S_t r_t,
// with the same modes as the 64-wide chunked forward: dense or segment
// (resolve_unit), initial state or zero, final state, and a state checkpoint
// at every 16th token of a sequence (the state entering tokens 0, 16, 32...).
//
// One workgroup of 256 lanes (four waves) per (sequence, head). In wave v,
// lane l holds key quarter l / 16 (32 keys) of the two state rows
// 32 v + l % 16 + 16 m, m = 0..1, so every row value a lane reads serves two
// state rows; the four key quarters of a row add their partial dot products
// with register swaps between the wave's 16-lane rows. Four waves of 64
// elements per lane run two waves per SIMD at the prefill shape (512 units
// on 256 CUs), against one for two waves of 128 elements: 1.59 against 2.25
// ms. The r, w, k, a, b rows of a block of tokens (8 for 16-bit streams, 4
// for fp32) are staged in LDS as fp32 (w already exponentiated when it holds
// log(decay)), double-buffered with the next block's loads in flight, and
// read as 16-byte broadcasts, one address per key quarter; the quarters'
// 16-byte chunks alternate in a row so that the four addresses fall in
// different banks. Per token and lane: 64 multiply-adds for the rows' S a,
// 3 x 64 for their update and 64 for S r, against 40 broadcasts per wave.
#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename TI>
__device__ __forceinline__ void unpack(const u32x4 &x, float *out);

// The lanes are copied to plain words first: bit-casting a vector element
// expression directly (x.y) yields the vector's first element with this
// compiler.
template <>
__device__ __forceinline__ void unpack<float>(const u32x4 &x, float *out) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = __builtin_bit_cast(float, w[e]);
}

template <>
__device__ __forceinline__ void unpack<uint16_t>(const u32x4 &x, float *out) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        out[2 * e] = __builtin_bit_cast(float, w[e] << 16);
        out[2 * e + 1] = __builtin_bit_cast(float, w[e] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void unpack<_Float16>(const u32x4 &x, float *out) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        out[2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xFFFFu));
        out[2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
    }
}

template <typename TI>
__global__ __launch_bounds__(256) void fwd128_kernel(FwdArgs p) {
    constexpr int N = 128;
    constexpr int EPL = 16 / (int)sizeof(TI);        // elements per 16-byte load
    constexpr int TB = sizeof(TI) == 2 ? 8 : 4;      // tokens per staged block
    constexpr int CPR = N / EPL;                     // 16-byte chunks per row
    constexpr int NT = 256;                          // threads
    constexpr int TOTAL = TB * 5 * CPR;              // 16-byte chunks per block
    constexpr int LOADS = (TOTAL + NT - 1) / NT;     // loads per lane and block
    __shared__ __align__(16) float vec[2][TB][5][N];  // [buffer][token][r w k a b][N]

    const int H = p.seg.H;
    const int64_t unit = blockIdx.x;
    const int sq = (int)(unit / H), h = (int)(unit % H);
    const Unit u = resolve_unit(p.seg, sq);
    constexpr int RPL = 2, KL = 32, NQ = KL / 4;        // rows per lane, keys per lane, quads
    const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
    const int kq = ln >> 4;                          // key quarter: keys [32 kq, 32 kq + 32)
    const int rb = wv * 32 + (ln & 15);              // the lane's rows: rb + 16 m, m = 0..1
    const int64_t ts = (int64_t)H * N;               // stream pitch of one token
    const int64_t srow = ((int64_t)unit * N + rb) * N + kq * KL;

    float S[RPL][KL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        if (p.s0) {
#pragma unroll
            for (int j = 0; j < KL; j += 4) {
                const f32x4 x = *(const f32x4 *)(p.s0 + srow + 16 * m * N + j);
                S[m][j] = x.x; S[m][j + 1] = x.y; S[m][j + 2] = x.z; S[m][j + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < KL; ++j) S[m][j] = 0.f;
        }
    }
    const TI *src[5] = {(const TI *)p.r, (const TI *)p.w, (const TI *)p.k, (const TI *)p.a, (const TI *)p.b};

    u32x4 st[LOADS];
    // chunk c = q*N + tid of a block: token c / (5*CPR), row (c / CPR) % 5, chunk c % CPR;
    // tokens past the sequence are clamped to its last token
#define F128_LOAD(t0)                                                                       \
    do {                                                                                    \
        _Pragma("unroll") for (int q = 0; q < LOADS; ++q) {                                 \
            const int c = q * NT + tid;                                                     \
            if (c >= TOTAL) break;                                                          \
            const int tt = c / (5 * CPR), row = (c / CPR) % 5, ch = c % CPR;                \
            const int64_t tok = u.start + min((t0) + tt, u.len - 1);                        \
            const TI *s_ = row == 0 ? src[0] : row == 1 ? src[1] : row == 2 ? src[2]        \
                         : row == 3 ? src[3] : src[4];                                      \
            st[q] = *(const u32x4 *)(s_ + tok * ts + h * N + ch * EPL);                     \
        }                                                                                   \
    } while (0)
    // element f of a staged row sits at 4 * slot(f / 4) + f % 4, where the
    // 16-byte chunk c of key quarter c / 8 goes to slot 4 (c % 8) + c / 8
#define F128_STORE(buf)                                                                     \
    do {                                                                                    \
        _Pragma("unroll") for (int q = 0; q < LOADS; ++q) {                                 \
            const int c = q * NT + tid;                                                     \
            if (c >= TOTAL) break;                                                          \
            const int tt = c / (5 * CPR), row = (c / CPR) % 5, ch = c % CPR;                \
            float x[EPL];                                                                   \
            unpack<TI>(st[q], x);                                                           \
            if (row == 1 && p.logw) {                                                       \
                _Pragma("unroll") for (int e = 0; e < EPL; ++e) x[e] = expf(x[e]);          \
            }                                                                               \
            float *d_ = vec[buf][tt][row];                                                  \
            _Pragma("unroll") for (int e = 0; e < EPL; e += 4) {                            \
                const int c4 = (ch * EPL + e) >> 2;                                         \
                *(f32x4 *)(d_ + 4 * (4 * (c4 & 7) + (c4 >> 3))) =                           \
                    f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};                              \
            }                                                                               \
        }                                                                                   \
    } while (0)

    const int len = u.len;
    if (len > 0) {
        F128_LOAD(0);
        F128_STORE(0);
    }
    __syncthreads();
    const int nblk = (len + TB - 1) / TB;
    for (int blk = 0; blk < nblk; ++blk) {
        const int buf = blk & 1, t0 = blk * TB;
        if (blk + 1 < nblk) F128_LOAD(t0 + TB);
        const int tn = min(TB, len - t0);
        for (int tt = 0; tt < tn; ++tt) {
            const int t = t0 + tt;
            const int64_t tok = u.start + t;
            if (p.ckpt && (t % kChunk) == 0) {
                float *c = p.ckpt + ((u.ckpt + t / kChunk) * H + h) * (int64_t)(N * N) + (int64_t)rb * N + kq * KL;
#pragma unroll
                for (int m = 0; m < RPL; ++m)
#pragma unroll
                    for (int j = 0; j < KL; j += 4)
                        *(f32x4 *)(c + 16 * m * N + j) = f32x4{S[m][j], S[m][j + 1], S[m][j + 2], S[m][j + 3]};
            }
            // the lane's key quarter: quad q of it at 16 q floats from here
            const float *rr = vec[buf][tt][0] + 4 * kq, *wr = vec[buf][tt][1] + 4 * kq;
            const float *kr = vec[buf][tt][2] + 4 * kq, *ar = vec[buf][tt][3] + 4 * kq;
            const float *br = vec[buf][tt][4] + 4 * kq;
            float vv[RPL], x[RPL];
#pragma unroll
            for (int m = 0; m < RPL; ++m) vv[m] = IO<TI>::ld((const TI *)p.v, tok * ts + h * N + rb + 16 * m);
            float pa[RPL][2];
#pragma unroll
            for (int m = 0; m < RPL; ++m) pa[m][0] = pa[m][1] = 0.f;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 a4 = *(const f32x4 *)(ar + 16 * q);
                const int j = 4 * q;
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    pa[m][0] = fmaf(S[m][j], a4.x, pa[m][0]);
                    pa[m][1] = fmaf(S[m][j + 1], a4.y, pa[m][1]);
                    pa[m][0] = fmaf(S[m][j + 2], a4.z, pa[m][0]);
                    pa[m][1] = fmaf(S[m][j + 3], a4.w, pa[m][1]);
                }
            }
#pragma unroll
            for (int m = 0; m < RPL; ++m) x[m] = pa[m][0] + pa[m][1];
            {   // over the four key quarters (lane rows): rows 0, 2 of lanes
                // end with x0's total, rows 1, 3 with x1's, then both to all
                float a0 = x[0], a1 = x[1];
                swap16(a0, a1);
                float y = a0 + a1, y2 = y;
                swap32(y, y2);
                float t = y + y2, t2 = t;
                swap16(t, t2);
                x[0] = t; x[1] = t2;
            }
            float py[RPL][2];
#pragma unroll
            for (int m = 0; m < RPL; ++m) py[m][0] = py[m][1] = 0.f;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 w4 = *(const f32x4 *)(wr + 16 * q), b4 = *(const f32x4 *)(br + 16 * q);
                const f32x4 k4 = *(const f32x4 *)(kr + 16 * q), r4 = *(const f32x4 *)(rr + 16 * q);
                const int j = 4 * q;
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    S[m][j] = fmaf(S[m][j], w4.x, fmaf(x[m], b4.x, vv[m] * k4.x));
                    S[m][j + 1] = fmaf(S[m][j + 1], w4.y, fmaf(x[m], b4.y, vv[m] * k4.y));
                    S[m][j + 2] = fmaf(S[m][j + 2], w4.z, fmaf(x[m], b4.z, vv[m] * k4.z));
                    S[m][j + 3] = fmaf(S[m][j + 3], w4.w, fmaf(x[m], b4.w, vv[m] * k4.w));
                    py[m][0] = fmaf(S[m][j], r4.x, py[m][0]);
                    py[m][1] = fmaf(S[m][j + 1], r4.y, py[m][1]);
                    py[m][0] = fmaf(S[m][j + 2], r4.z, py[m][0]);
                    py[m][1] = fmaf(S[m][j + 3], r4.w, py[m][1]);
                }
            }
            float o[RPL];
#pragma unroll
            for (int m = 0; m < RPL; ++m) o[m] = py[m][0] + py[m][1];
            // key quarter m holds row rb + 16 m's total and writes it: 64
            // consecutive outputs per wave
            float om;
            {
                float a0 = o[0], a1 = o[1];
                swap16(a0, a1);
                float y = a0 + a1, y2 = y;
                swap32(y, y2);
                om = y + y2;                       // rows 0, 2: o0's total; rows 1, 3: o1's
            }
            if (kq < RPL) IO<TI>::st((TI *)p.y, tok * ts + h * N + rb + 16 * kq, om);
        }
        if (blk + 1 < nblk) F128_STORE(buf ^ 1);
        __syncthreads();
    }
#undef F128_LOAD
#undef F128_STORE
    if (p.s_out) {
#pragma unroll
        for (int m = 0; m < RPL; ++m)
#pragma unroll
            for (int j = 0; j < KL; j += 4)
                *(f32x4 *)(p.s_out + srow + 16 * m * N + j) = f32x4{S[m][j], S[m][j + 1], S[m][j + 2], S[m][j + 3]};
    }
}

template <typename TI>
hipError_t launch_t(const FwdArgs &a, int64_t units, hipStream_t stream) {
    hipLaunchKernelGGL(fwd128_kernel<TI>, dim3((unsigned)units), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward128(const FwdArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)(a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B) * a.seg.H;
    if (a.dtype == 1) return launch_t<uint16_t>(a, units, stream);
    if (a.dtype == 2) return launch_t<_Float16>(a, units, stream);
    return launch_t<float>(a, units, stream);
}

}  // namespace wkv7
