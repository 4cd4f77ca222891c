// WKV-7 forward at head size 128 (the matched head size of the rwkv-lab
// page's GDN conversion target), token by token:
//     S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T + v_t k_t^T,   y_t = S_t r_t,
// with the same modes as the 64-wide chunked forward: dense or segment
// (resolve_unit), initial state or zero, final state, and a state checkpoint
// at every 16th token of a sequence (the state entering tokens 0, 16, 32...).
//
// One workgroup of 128 lanes (two waves) per (sequence, head). In wave v,
// lane l holds key half l / 32 (64 keys) of state rows 64 v + l % 32 and
// 64 v + l % 32 + 32, so every row value a lane reads serves two state rows;
// the two key halves of a row add their partial dot products with one lane
// exchange inside the wave. The r, w, k, a, b rows of a block of tokens (16
// for 16-bit streams, 8 for fp32) are staged in LDS as fp32 (w already
// exponentiated when it holds log(decay)), double-buffered with the next
// block's loads in flight, and read as 16-byte broadcasts, one address per
// key half; the halves' 16-byte chunks alternate in a row so that the two
// addresses fall in different banks. Per token and lane: 128 multiply-adds
// for the two rows' S a, 3 x 128 for their update and 128 for S r, against 80
// broadcasts per wave.
#include "wkv7_kernels.h"

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
__global__ __launch_bounds__(128) void fwd128_kernel(FwdArgs p) {
    constexpr int N = 128;
    constexpr int EPL = 16 / (int)sizeof(TI);        // elements per 16-byte load
    constexpr int TB = sizeof(TI) == 2 ? 8 : 4;      // tokens per staged block
    constexpr int CPR = N / EPL;                     // 16-byte chunks per row
    constexpr int LOADS = TB * 5 * CPR / N;          // loads per lane and block
    static_assert(TB * 5 * CPR % N == 0, "whole loads per lane");
    __shared__ __align__(16) float vec[2][TB][5][N];  // [buffer][token][r w k a b][N]

    const int H = p.seg.H;
    const int64_t unit = blockIdx.x;
    const int sq = (int)(unit / H), h = (int)(unit % H);
    const Unit u = resolve_unit(p.seg, sq);
    const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
    const int kh = ln >> 5;                          // key half: keys [64 kh, 64 kh + 64)
    const int i0 = wv * 64 + (ln & 31), i1 = i0 + 32; // the lane's two state rows
    const int64_t ts = (int64_t)H * N;               // stream pitch of one token
    const int64_t srow0 = ((int64_t)unit * N + i0) * N + kh * 64;
    const int64_t srow1 = srow0 + 32 * N;

    float S0[64], S1[64];
    if (p.s0) {
#pragma unroll
        for (int j = 0; j < 64; j += 4) {
            const f32x4 x = *(const f32x4 *)(p.s0 + srow0 + j);
            S0[j] = x.x; S0[j + 1] = x.y; S0[j + 2] = x.z; S0[j + 3] = x.w;
            const f32x4 z = *(const f32x4 *)(p.s0 + srow1 + j);
            S1[j] = z.x; S1[j + 1] = z.y; S1[j + 2] = z.z; S1[j + 3] = z.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 64; ++j) S0[j] = S1[j] = 0.f;
    }
    const TI *src[5] = {(const TI *)p.r, (const TI *)p.w, (const TI *)p.k, (const TI *)p.a, (const TI *)p.b};

    u32x4 st[LOADS];
    // chunk c = q*N + tid of a block: token c / (5*CPR), row (c / CPR) % 5, chunk c % CPR;
    // tokens past the sequence are clamped to its last token
#define F128_LOAD(t0)                                                                       \
    do {                                                                                    \
        _Pragma("unroll") for (int q = 0; q < LOADS; ++q) {                                 \
            const int c = q * N + tid;                                                      \
            const int tt = c / (5 * CPR), row = (c / CPR) % 5, ch = c % CPR;                \
            const int64_t tok = u.start + min((t0) + tt, u.len - 1);                        \
            const TI *s_ = row == 0 ? src[0] : row == 1 ? src[1] : row == 2 ? src[2]        \
                         : row == 3 ? src[3] : src[4];                                      \
            st[q] = *(const u32x4 *)(s_ + tok * ts + h * N + ch * EPL);                     \
        }                                                                                   \
    } while (0)
    // element f of a staged row sits at 4 * slot(f / 4) + f % 4, where the
    // 16-byte chunk c of key half c / 16 goes to slot 2 (c % 16) + c / 16
#define F128_STORE(buf)                                                                     \
    do {                                                                                    \
        _Pragma("unroll") for (int q = 0; q < LOADS; ++q) {                                 \
            const int c = q * N + tid;                                                      \
            const int tt = c / (5 * CPR), row = (c / CPR) % 5, ch = c % CPR;                \
            float x[EPL];                                                                   \
            unpack<TI>(st[q], x);                                                           \
            if (row == 1 && p.logw) {                                                       \
                _Pragma("unroll") for (int e = 0; e < EPL; ++e) x[e] = expf(x[e]);          \
            }                                                                               \
            float *d_ = vec[buf][tt][row];                                                  \
            _Pragma("unroll") for (int e = 0; e < EPL; e += 4) {                            \
                const int c4 = (ch * EPL + e) >> 2;                                         \
                *(f32x4 *)(d_ + 4 * (2 * (c4 & 15) + (c4 >> 4))) =                          \
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
                float *c = p.ckpt + ((u.ckpt + t / kChunk) * H + h) * (int64_t)(N * N) + (int64_t)i0 * N + kh * 64;
#pragma unroll
                for (int j = 0; j < 64; j += 4) {
                    *(f32x4 *)(c + j) = f32x4{S0[j], S0[j + 1], S0[j + 2], S0[j + 3]};
                    *(f32x4 *)(c + 32 * N + j) = f32x4{S1[j], S1[j + 1], S1[j + 2], S1[j + 3]};
                }
            }
            // the lane's key half: quad q of it at 8 q floats from here
            const float *rr = vec[buf][tt][0] + 4 * kh, *wr = vec[buf][tt][1] + 4 * kh;
            const float *kr = vec[buf][tt][2] + 4 * kh, *ar = vec[buf][tt][3] + 4 * kh;
            const float *br = vec[buf][tt][4] + 4 * kh;
            const float v0 = IO<TI>::ld((const TI *)p.v, tok * ts + h * N + i0);
            const float v1 = IO<TI>::ld((const TI *)p.v, tok * ts + h * N + i1);
            float p0[4] = {0.f, 0.f, 0.f, 0.f}, p1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const f32x4 a4 = *(const f32x4 *)(ar + 8 * q);
                const int j = 4 * q;
                p0[0] = fmaf(S0[j], a4.x, p0[0]);
                p0[1] = fmaf(S0[j + 1], a4.y, p0[1]);
                p0[2] = fmaf(S0[j + 2], a4.z, p0[2]);
                p0[3] = fmaf(S0[j + 3], a4.w, p0[3]);
                p1[0] = fmaf(S1[j], a4.x, p1[0]);
                p1[1] = fmaf(S1[j + 1], a4.y, p1[1]);
                p1[2] = fmaf(S1[j + 2], a4.z, p1[2]);
                p1[3] = fmaf(S1[j + 3], a4.w, p1[3]);
            }
            float x0 = (p0[0] + p0[1]) + (p0[2] + p0[3]);
            float x1 = (p1[0] + p1[1]) + (p1[2] + p1[3]);
            x0 += __shfl_xor(x0, 32);
            x1 += __shfl_xor(x1, 32);
            float y0[4] = {0.f, 0.f, 0.f, 0.f}, y1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const f32x4 w4 = *(const f32x4 *)(wr + 8 * q), b4 = *(const f32x4 *)(br + 8 * q);
                const f32x4 k4 = *(const f32x4 *)(kr + 8 * q), r4 = *(const f32x4 *)(rr + 8 * q);
                const int j = 4 * q;
                S0[j] = fmaf(S0[j], w4.x, fmaf(x0, b4.x, v0 * k4.x));
                S0[j + 1] = fmaf(S0[j + 1], w4.y, fmaf(x0, b4.y, v0 * k4.y));
                S0[j + 2] = fmaf(S0[j + 2], w4.z, fmaf(x0, b4.z, v0 * k4.z));
                S0[j + 3] = fmaf(S0[j + 3], w4.w, fmaf(x0, b4.w, v0 * k4.w));
                S1[j] = fmaf(S1[j], w4.x, fmaf(x1, b4.x, v1 * k4.x));
                S1[j + 1] = fmaf(S1[j + 1], w4.y, fmaf(x1, b4.y, v1 * k4.y));
                S1[j + 2] = fmaf(S1[j + 2], w4.z, fmaf(x1, b4.z, v1 * k4.z));
                S1[j + 3] = fmaf(S1[j + 3], w4.w, fmaf(x1, b4.w, v1 * k4.w));
                y0[0] = fmaf(S0[j], r4.x, y0[0]);
                y0[1] = fmaf(S0[j + 1], r4.y, y0[1]);
                y0[2] = fmaf(S0[j + 2], r4.z, y0[2]);
                y0[3] = fmaf(S0[j + 3], r4.w, y0[3]);
                y1[0] = fmaf(S1[j], r4.x, y1[0]);
                y1[1] = fmaf(S1[j + 1], r4.y, y1[1]);
                y1[2] = fmaf(S1[j + 2], r4.z, y1[2]);
                y1[3] = fmaf(S1[j + 3], r4.w, y1[3]);
            }
            float o0 = (y0[0] + y0[1]) + (y0[2] + y0[3]);
            float o1 = (y1[0] + y1[1]) + (y1[2] + y1[3]);
            o0 += __shfl_xor(o0, 32);
            o1 += __shfl_xor(o1, 32);
            // key half 0 writes row i0, key half 1 row i1: 64 consecutive outputs per wave
            IO<TI>::st((TI *)p.y, tok * ts + h * N + (kh ? i1 : i0), kh ? o1 : o0);
        }
        if (blk + 1 < nblk) F128_STORE(buf ^ 1);
        __syncthreads();
    }
#undef F128_LOAD
#undef F128_STORE
    if (p.s_out) {
#pragma unroll
        for (int j = 0; j < 64; j += 4) {
            *(f32x4 *)(p.s_out + srow0 + j) = f32x4{S0[j], S0[j + 1], S0[j + 2], S0[j + 3]};
            *(f32x4 *)(p.s_out + srow1 + j) = f32x4{S1[j], S1[j + 1], S1[j + 2], S1[j + 3]};
        }
    }
}

template <typename TI>
hipError_t launch_t(const FwdArgs &a, int64_t units, hipStream_t stream) {
    hipLaunchKernelGGL(fwd128_kernel<TI>, dim3((unsigned)units), dim3(128), 0, stream, a);
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
