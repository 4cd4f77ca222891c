// WKV-7 forward at head size 128 (the matched head size of the rwkv-lab
// page's GDN conversion target), token by token:
//     S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T + v_t k_t^T,   y_t = S_t r_t,
// with the same modes as the 64-wide chunked forward: dense or segment
// (resolve_unit), initial state or zero, final state, and a state checkpoint
// at every 16th token of a sequence (the state entering tokens 0, 16, 32...).
//
// One workgroup of 128 lanes per (sequence, head): lane i holds state row i
// in 128 registers. The r, w, k, a, b rows of a block of tokens (16 for
// 16-bit streams, 8 for fp32) are staged in LDS as fp32 (w already
// exponentiated when it holds log(decay)), double-buffered with the next
// block's loads in flight, and read by every lane as 16-byte broadcasts.
// Per token and lane: 128 multiply-adds for S_i a, 3 x 128 for the update and
// 128 for S_i r. LDS broadcasts (160 per token and wave) bound the kernel.
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
    constexpr int TB = sizeof(TI) == 2 ? 16 : 8;     // tokens per staged block
    constexpr int CPR = N / EPL;                     // 16-byte chunks per row
    constexpr int LOADS = TB * 5 * CPR / N;          // loads per lane and block
    static_assert(TB * 5 * CPR % N == 0, "whole loads per lane");
    __shared__ __align__(16) float vec[2][TB][5][N];  // [buffer][token][r w k a b][N]

    const int H = p.seg.H;
    const int64_t unit = blockIdx.x;
    const int sq = (int)(unit / H), h = (int)(unit % H);
    const Unit u = resolve_unit(p.seg, sq);
    const int i = threadIdx.x;
    const int64_t ts = (int64_t)H * N;               // stream pitch of one token
    const int64_t srow = ((int64_t)unit * N + i) * N;

    float S[N];
    if (p.s0) {
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            const f32x4 x = *(const f32x4 *)(p.s0 + srow + j);
            S[j] = x.x; S[j + 1] = x.y; S[j + 2] = x.z; S[j + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) S[j] = 0.f;
    }
    const TI *src[5] = {(const TI *)p.r, (const TI *)p.w, (const TI *)p.k, (const TI *)p.a, (const TI *)p.b};

    u32x4 st[LOADS];
    // chunk c = q*N + i of a block: token c / (5*CPR), row (c / CPR) % 5, chunk c % CPR;
    // tokens past the sequence are clamped to its last token
#define F128_LOAD(t0)                                                                       \
    do {                                                                                    \
        _Pragma("unroll") for (int q = 0; q < LOADS; ++q) {                                 \
            const int c = q * N + i;                                                        \
            const int tt = c / (5 * CPR), row = (c / CPR) % 5, ch = c % CPR;                \
            const int64_t tok = u.start + min((t0) + tt, u.len - 1);                        \
            const TI *s_ = row == 0 ? src[0] : row == 1 ? src[1] : row == 2 ? src[2]        \
                         : row == 3 ? src[3] : src[4];                                      \
            st[q] = *(const u32x4 *)(s_ + tok * ts + h * N + ch * EPL);                     \
        }                                                                                   \
    } while (0)
#define F128_STORE(buf)                                                                     \
    do {                                                                                    \
        _Pragma("unroll") for (int q = 0; q < LOADS; ++q) {                                 \
            const int c = q * N + i;                                                        \
            const int tt = c / (5 * CPR), row = (c / CPR) % 5, ch = c % CPR;                \
            float x[EPL];                                                                   \
            unpack<TI>(st[q], x);                                                           \
            if (row == 1 && p.logw) {                                                       \
                _Pragma("unroll") for (int e = 0; e < EPL; ++e) x[e] = expf(x[e]);          \
            }                                                                               \
            float *d_ = &vec[buf][tt][row][ch * EPL];                                       \
            _Pragma("unroll") for (int e = 0; e < EPL; e += 4)                              \
                *(f32x4 *)(d_ + e) = f32x4{x[e], x[e + 1], x[e + 2], x[e + 3]};             \
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
                float *c = p.ckpt + ((u.ckpt + t / kChunk) * H + h) * (int64_t)(N * N) + (int64_t)i * N;
#pragma unroll
                for (int j = 0; j < N; j += 4) *(f32x4 *)(c + j) = f32x4{S[j], S[j + 1], S[j + 2], S[j + 3]};
            }
            const float *rr = vec[buf][tt][0], *wr = vec[buf][tt][1], *kr = vec[buf][tt][2];
            const float *ar = vec[buf][tt][3], *br = vec[buf][tt][4];
            const float vi = IO<TI>::ld((const TI *)p.v, tok * ts + h * N + i);
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < N; j += 4) {
                const f32x4 a4 = *(const f32x4 *)(ar + j);
                s4[0] = fmaf(S[j], a4.x, s4[0]);
                s4[1] = fmaf(S[j + 1], a4.y, s4[1]);
                s4[2] = fmaf(S[j + 2], a4.z, s4[2]);
                s4[3] = fmaf(S[j + 3], a4.w, s4[3]);
            }
            const float sa = (s4[0] + s4[1]) + (s4[2] + s4[3]);
            float y4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < N; j += 4) {
                const f32x4 w4 = *(const f32x4 *)(wr + j), b4 = *(const f32x4 *)(br + j);
                const f32x4 k4 = *(const f32x4 *)(kr + j), r4 = *(const f32x4 *)(rr + j);
                S[j] = fmaf(S[j], w4.x, fmaf(sa, b4.x, vi * k4.x));
                S[j + 1] = fmaf(S[j + 1], w4.y, fmaf(sa, b4.y, vi * k4.y));
                S[j + 2] = fmaf(S[j + 2], w4.z, fmaf(sa, b4.z, vi * k4.z));
                S[j + 3] = fmaf(S[j + 3], w4.w, fmaf(sa, b4.w, vi * k4.w));
                y4[0] = fmaf(S[j], r4.x, y4[0]);
                y4[1] = fmaf(S[j + 1], r4.y, y4[1]);
                y4[2] = fmaf(S[j + 2], r4.z, y4[2]);
                y4[3] = fmaf(S[j + 3], r4.w, y4[3]);
            }
            IO<TI>::st((TI *)p.y, tok * ts + h * N + i, (y4[0] + y4[1]) + (y4[2] + y4[3]));
        }
        if (blk + 1 < nblk) F128_STORE(buf ^ 1);
        __syncthreads();
    }
#undef F128_LOAD
#undef F128_STORE
    if (p.s_out) {
#pragma unroll
        for (int j = 0; j < N; j += 4) *(f32x4 *)(p.s_out + srow + j) = f32x4{S[j], S[j + 1], S[j + 2], S[j + 3]};
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
