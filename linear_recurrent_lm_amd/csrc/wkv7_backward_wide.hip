// WKV-7 backward at head size 128, token by token, from the 16-token state
// checkpoints of the forward. Reverse-mode through
//     S_t = S_{t-1} diag(w_t) + (S_{t-1} a_t) b_t^T + v_t k_t^T,   y_t = S_t r_t
// with dS the gradient of the state after token t (ds_out after the last):
//     dS += dy_t r_t^T;                 dr_t = S_t^T dy_t
//     dv_t = dS k_t;   dk_t = dS^T v_t;  dsa = dS b_t;   db_t = dS^T sa_t
//     dw_t = colsum(dS o S_{t-1});       da_t = S_{t-1}^T dsa
//     dS <- dS diag(w_t) + dsa a_t^T    (the gradient of the state before t)
// where sa_t = S_{t-1} a_t. S_{t-1} is never rebuilt from S_t (that divides by
// w): the states are recomputed forward from the chunk's checkpoint.
//
// One 1024-thread workgroup owns a whole (sequence, head). Thread t holds the
// 4 x 4 block of the state and of dS at value rows 4 (t / 32) .. + 3 and keys
// 4 (t % 32) .. + 3, so a row spreads over the 32 lanes of a half-wave and a
// key over the 32 half-waves.
// - Row sums (S a, dS k, dS b) add the thread's 4 keys, then reduce over the
//   half-wave with register-to-register lane exchanges (no LDS).
// - Key sums (the five key-indexed gradients dr, dk, db, dw, da over all 128
//   rows) add the thread's 4 rows, swap halves of their 20 values with the
//   other half-wave (each half keeps 10 and adds the partner's), and the 16
//   waves' partial sums meet in LDS, where 640 threads add them and write the
//   gradients. The partial-sum area is double-buffered by token, so one
//   barrier per token separates its writes from the sums.
// Nothing is accumulated across workgroups: every gradient element is written
// once, in its own dtype, and the result does not depend on scheduling.
//
// States: a chunk is walked back in segments of kSeg tokens. Each segment
// starts from the chunk's checkpoint (re-read; it stays in L2), steps forward
// to the segment's first token without storing, then keeps the states before
// each of its tokens in registers for the reverse pass (2.5 forward steps per
// token for kSeg = 4). Those states enter only their token's own gradients
// (dr, dw, da), never the recursion of dS, so with bf16 streams and bf16
// gradients they are kept as bf16 pairs, half the registers, and a segment
// spans 8 tokens (1.5 forward steps per token); the recomputed chain itself
// stays fp32.
#include <type_traits>

#include "wkv7_kernels.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr int kWN = 128;              // head size
constexpr int kWThreads = 1024;
constexpr int kSeg = 4;               // tokens per recompute segment
constexpr int kSegHS = 8;             // the same with the segment's states in bf16
enum { SW = 0, SA, SB, SK, SR, NSTAGE };     // staged key-indexed rows
enum { GR = 0, GK, GB, GW, GA, NGRAD };      // key-indexed gradients

// LDS (floats): staged rows [NSTAGE][16][128] (w exponentiated for log
// input), v and dy by value row [2][16][128], S a of each token [16][128],
// and the key sums' partial-sum area [2 buffers][16 waves][20 x 32].
constexpr int L_ST = 0;
constexpr int L_VD = L_ST + NSTAGE * kChunk * kWN;
constexpr int L_SAV = L_VD + 2 * kChunk * kWN;
constexpr int L_PART = L_SAV + kChunk * kWN;
constexpr int kPartWave = 20 * 32;
constexpr int L_TOTAL = L_PART + 2 * 16 * kPartWave;
static_assert(L_TOTAL * 4 <= 160 * 1024, "LDS budget");

// Partial-sum slot of value v (0..19) of key group kq: the 32 key groups of a
// value are consecutive, XOR-swizzled so that the summing threads (32
// consecutive keys: 8 key groups x 4 values) hit 32 distinct banks.
__device__ __forceinline__ int part_slot(int v, int kq) { return v * 32 + (kq ^ (8 * (v & 3))); }
// Which value v holds gradient g of key 4 kq + e after the half-wave swap:
// the lower half keeps dr, dk and db of keys e = 0, 1; the upper half dw, da
// and db of keys e = 2, 3.
__device__ __forceinline__ int grad_value(int g, int e) {
    return g == GR ? e : g == GK ? 4 + e : g == GB ? (e < 2 ? 8 + e : 16 + e) : g == GW ? 10 + e : 14 + e;
}

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

// x[r]: this thread's partial sums (its 4 keys) of rows 4 (t / 32) + r; on
// return, the sums over all 128 keys, in every lane of the half-wave. The
// half-wave's even 16-lane row keeps rows 0, 1 and its odd row rows 2, 3,
// each adding the other row's share; each row of lanes sums its two, then two
// swaps hand every lane all four.
__device__ __forceinline__ void row_sums(float (&x)[4], int lane) {
    float a0 = x[0], a2 = x[2], a1 = x[1], a3 = x[3];
    swap16(a0, a2);
    swap16(a1, a3);
    float k0 = sum16(a0 + a2), k1 = sum16(a1 + a3);   // even row: rows 0, 1; odd row: rows 2, 3
    float g1a = k0, g1b = k1, g2a = k1, g2b = k0;
    swap16(g1a, g1b);                                  // even: rows 0, 2; odd: rows 1, 3
    swap16(g2a, g2b);                                  // even: rows 1, 3; odd: rows 0, 2
    const bool odd = (lane & 16) != 0;
    x[0] = odd ? g2a : g1a;
    x[1] = odd ? g1a : g2a;
    x[2] = odd ? g2b : g1b;
    x[3] = odd ? g1b : g2b;
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kWThreads, 1) void bwd128_kernel(BwdArgs p, int32_t units) {
    extern __shared__ __align__(16) float sm[];
    // bf16 streams with bf16 gradients: the states before the tokens of a
    // segment are held as bf16 pairs, so a segment spans 8 tokens
    constexpr bool kHS = std::is_same<TI, uint16_t>::value && std::is_same<TO, uint16_t>::value;
    constexpr int kSegT = kHS ? kSegHS : kSeg;
    const int unit = blockIdx.x;
    if (unit >= units) return;
    const int H = p.seg.H;
    const int h = unit % H, sq = unit / H;
    const Unit u = resolve_unit(p.seg, sq);
    // The thread indices are re-derived from an opaque copy of the thread id
    // in each phase, so that the many addresses built from them are formed
    // where they are used instead of being hoisted out of the loops and kept
    // live (or spilled) throughout.
    int tid, wave, lane, hf, kq, row0, key0;
    auto relane = [&]() {
        int x = (int)threadIdx.x;
        asm volatile("" : "+v"(x));
        tid = x; wave = x >> 6; lane = x & 63; hf = lane >> 5; kq = lane & 31;
        row0 = 4 * (2 * wave + hf); key0 = 4 * kq;
    };
    relane();
    const int64_t ts = (int64_t)H * kWN;            // token pitch of a stream
    const int64_t base = (u.start * H + h) * kWN;
    const int64_t sbase = ((int64_t)sq * H + h) * (int64_t)(kWN * kWN);
    const int nch = (u.len + kChunk - 1) / kChunk;

    // dS: rows row0 .. + 3, keys key0 .. + 3 (element 4 r + e)
    float dS[16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.ds_out) x = *(const float4 *)(p.ds_out + sbase + (int64_t)(row0 + r) * kWN + key0);
        dS[4 * r] = x.x; dS[4 * r + 1] = x.y; dS[4 * r + 2] = x.z; dS[4 * r + 3] = x.w;
    }

    auto keyrow = [&](int s, int e) { return *(const float4 *)(sm + L_ST + (s * kChunk + e) * kWN + key0); };
    auto valrow = [&](int s, int e) { return *(const float4 *)(sm + L_VD + (s * kChunk + e) * kWN + row0); };
    // one forward step of this thread's 16 elements; sa = S a of its rows
    auto step = [&](float (&S)[16], int e, float (&sa)[4]) {
        const float4 w4 = keyrow(SW, e), a4 = keyrow(SA, e), b4 = keyrow(SB, e), k4 = keyrow(SK, e);
        const float4 v4 = valrow(0, e);
        const float w[4] = {w4.x, w4.y, w4.z, w4.w}, b[4] = {b4.x, b4.y, b4.z, b4.w};
        const float k[4] = {k4.x, k4.y, k4.z, k4.w}, v[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
            sa[r] = fmaf(S[4 * r], a4.x, fmaf(S[4 * r + 1], a4.y, fmaf(S[4 * r + 2], a4.z, S[4 * r + 3] * a4.w)));
        row_sums(sa, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
                S[4 * r + e2] = fmaf(S[4 * r + e2], w[e2], fmaf(sa[r], b[e2], v[r] * k[e2]));
    };

    int buf = 0;
    // the reverse step of token e of the chunk starting at token t0, with P
    // the state before it
    auto token = [&](auto P, int e, int64_t t0) {
        relane();
        // operands are read where they are first used, to keep few live
        auto f4 = [](float4 x, float (&o)[4]) { o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w; };
        float dy[4], rr[4];
        f4(valrow(1, e), dy);
        f4(keyrow(SR, e), rr);
        float *part = sm + L_PART + (buf * 16 + wave) * kPartWave;
        // key sums of this thread's rows for two gradients: the lower half
        // keeps the first, the upper the second, each adding the partner's
        auto pair_out = [&](const float (&g1)[4], const float (&g2)[4], int v1, int v2) {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float lo = g1[e2], hi = g2[e2];
                swap32(lo, hi);                         // lower half: both g1; upper: both g2
                part[part_slot((hf ? v2 : v1) + e2, kq)] = lo + hi;
            }
        };
        // dS becomes the gradient of S_t: add dy_t r_t^T
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) dS[4 * r + e2] = fmaf(dy[r], rr[e2], dS[4 * r + e2]);
        float k[4], b[4];
        f4(keyrow(SK, e), k);
        f4(keyrow(SB, e), b);
        float dv[4], dsa[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dv[r] = fmaf(dS[4 * r], k[0], fmaf(dS[4 * r + 1], k[1], fmaf(dS[4 * r + 2], k[2], dS[4 * r + 3] * k[3])));
            dsa[r] = fmaf(dS[4 * r], b[0], fmaf(dS[4 * r + 1], b[1], fmaf(dS[4 * r + 2], b[2], dS[4 * r + 3] * b[3])));
        }
        row_sums(dv, lane);
        row_sums(dsa, lane);
        float w[4], v[4], sa[4];
        f4(keyrow(SW, e), w);
        f4(valrow(0, e), v);
        f4(*(const float4 *)(sm + L_SAV + e * kWN + row0), sa);
        {   // dr = S_t^T dy (S_t rebuilt from P), dw = colsum(dS o P)
            float gr[4], gw[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float x = 0.f, y = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float st = fmaf(P(4 * r + e2), w[e2], fmaf(sa[r], b[e2], v[r] * k[e2]));
                    x = fmaf(st, dy[r], x);
                    y = fmaf(dS[4 * r + e2], P(4 * r + e2), y);
                }
                gr[e2] = x;
                gw[e2] = y;
            }
            pair_out(gr, gw, grad_value(GR, 0), grad_value(GW, 0));
        }
        {   // dk = dS^T v, da = P^T dsa
            float gk[4], ga[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float x = 0.f, y = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x = fmaf(dS[4 * r + e2], v[r], x);
                    y = fmaf(P(4 * r + e2), dsa[r], y);
                }
                gk[e2] = x;
                ga[e2] = y;
            }
            pair_out(gk, ga, grad_value(GK, 0), grad_value(GA, 0));
        }
        {   // db = dS^T sa
            float gb[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float x = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) x = fmaf(dS[4 * r + e2], sa[r], x);
                gb[e2] = x;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float lo = gb[i], hi = gb[2 + i];
                swap32(lo, hi);                         // lower half: key i; upper: key 2 + i
                part[part_slot(hf ? grad_value(GB, 2 + i) : grad_value(GB, i), kq)] = lo + hi;
            }
        }
        // dv of the thread's rows: lanes 0-3 of each half write one row each
        if (kq < 4) {
            const float x = kq == 0 ? dv[0] : kq == 1 ? dv[1] : kq == 2 ? dv[2] : dv[3];
            IO<TO>::st((TO *)p.dv, base + (t0 + e) * ts + row0 + kq, x);
        }
        // the gradient of the state before token t
        float a[4];
        f4(keyrow(SA, e), a);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) dS[4 * r + e2] = fmaf(dS[4 * r + e2], w[e2], dsa[r] * a[e2]);
        __syncthreads();
        // the 16 waves' partial sums: thread f < 640 owns gradient f / 128 of key f % 128
        if (tid < NGRAD * kWN) {
            // g is uniform per wave: a scalar select of the output pointer (a
            // per-lane one loads it from the argument block with a vector
            // load, whose wait would also wait for every store in flight)
            const int g = __builtin_amdgcn_readfirstlane(tid >> 7), j = tid & 127;
            const float *q = sm + L_PART + buf * 16 * kPartWave + part_slot(grad_value(g, j & 3), j >> 2);
            float x = 0.f;
#pragma unroll
            for (int wv = 0; wv < 16; ++wv) x += q[wv * kPartWave];
            if (g == GW && p.logw) x *= sm[L_ST + (SW * kChunk + e) * kWN + j];   // d/d log(w) = w d/dw
            void *gp = g == GR ? p.dr : g == GK ? p.dk : g == GB ? p.db : g == GW ? p.dw : p.da;
            IO<TO>::st((TO *)gp, base + (t0 + e) * ts + j, x);
        }
        buf ^= 1;
    };

#pragma unroll 1
    for (int c = nch - 1; c >= 0; --c) {
        const int Lc = min(kChunk, u.len - c * kChunk);
        const int64_t t0 = (int64_t)c * kChunk;
        __syncthreads();                            // the previous chunk is done with the staged rows
        relane();
        // stage: items 0..1279 are 8 keys of the 5 key-indexed rows, items
        // 1280..1791 8 rows of v or dy; token rows clamped into the sequence
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = tid + it * kWThreads;
            if (i < NSTAGE * 256) {
                const int s = i >> 8, e = (i >> 4) & 15, g = i & 15;
                const TI *src = (const TI *)(s == SW ? p.w : s == SA ? p.a : s == SB ? p.b : s == SK ? p.k : p.r);
                Raw8<TI> raw;
                ld8(src + base + (t0 + min(e, Lc - 1)) * ts + 8 * g, raw);
                float x[8];
                un8(raw, x);
                if (s == SW) decay_of<8>(x, p.logw);
                float *d = sm + L_ST + (s * kChunk + e) * kWN + 8 * g;
                *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
                *(float4 *)(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
            } else if (i < NSTAGE * 256 + 512) {
                const int i2 = i - NSTAGE * 256;
                const int s = i2 >> 8, e = (i2 >> 4) & 15, g = i2 & 15;
                float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                const TI *src = (const TI *)(s == 0 ? p.v : p.dy);
                if (src) {
                    Raw8<TI> raw;
                    ld8(src + base + (t0 + min(e, Lc - 1)) * ts + 8 * g, raw);
                    un8(raw, x);
                }
                float *d = sm + L_VD + (s * kChunk + e) * kWN + 8 * g;
                *(float4 *)d = make_float4(x[0], x[1], x[2], x[3]);
                *(float4 *)(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
            }
        }
        __syncthreads();
        const float *ck = p.ckpt + ((u.ckpt + c) * H + h) * (int64_t)(kWN * kWN);
#pragma unroll 1
        for (int q = (Lc + kSegT - 1) / kSegT - 1; q >= 0; --q) {
            relane();
            float S[16];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float4 x = *(const float4 *)(ck + (int64_t)(row0 + r) * kWN + key0);
                S[4 * r] = x.x; S[4 * r + 1] = x.y; S[4 * r + 2] = x.z; S[4 * r + 3] = x.w;
            }
            float sa[4];
#pragma unroll 1
            for (int e = 0; e < kSegT * q; ++e) step(S, e, sa);
            // the states before each token of the segment, and their S a
            float Sp[kHS ? 1 : kSegT][16];
            uint32_t Sh[kHS ? kSegT : 1][8];
#pragma unroll
            for (int e = 0; e < kSegT; ++e) {
                const int te = kSegT * q + e;
                if (te < Lc) {
                    if constexpr (kHS) {
#pragma unroll
                        for (int x = 0; x < 8; ++x) Sh[e][x] = pk_bf16(S[2 * x], S[2 * x + 1]);
                    } else {
#pragma unroll
                        for (int x = 0; x < 16; ++x) Sp[e][x] = S[x];
                    }
                    step(S, te, sa);
                    *(float4 *)(sm + L_SAV + te * kWN + row0) = make_float4(sa[0], sa[1], sa[2], sa[3]);
                }
            }
#pragma unroll
            for (int e = kSegT - 1; e >= 0; --e) {
                const int te = kSegT * q + e;
                if (te < Lc) {
                    if constexpr (kHS) {
                        token([&](int x) { const uint32_t w2 = Sh[e][x >> 1]; return (x & 1) ? bf_hi(w2) : bf_lo(w2); },
                              te, t0);
                    } else {
                        token([&](int x) { return Sp[e][x]; }, te, t0);
                    }
                }
            }
        }
    }
    if (p.ds0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *(float4 *)(p.ds0 + sbase + (int64_t)(row0 + r) * kWN + key0) =
                make_float4(dS[4 * r], dS[4 * r + 1], dS[4 * r + 2], dS[4 * r + 3]);
    }
}

template <typename TI, typename TO>
hipError_t launch_t(const BwdArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)(a.seg.num_seqs > 0 ? a.seg.num_seqs : a.seg.B) * a.seg.H;
    const size_t lds = (size_t)L_TOTAL * sizeof(float);
    hipError_t e = hipFuncSetAttribute((const void *)bwd128_kernel<TI, TO>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd128_kernel<TI, TO>), dim3((unsigned)units), dim3(kWThreads), lds, stream, a,
                       (int32_t)units);
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_ti(const BwdArgs &a, hipStream_t stream) {
    if (a.grad_f32) return launch_t<TI, float>(a, stream);
    return launch_t<TI, TI>(a, stream);
}

}  // namespace

hipError_t launch_backward128(const BwdArgs &a, hipStream_t stream) {
    if (a.dtype == 1) return launch_ti<uint16_t>(a, stream);
    if (a.dtype == 2) return launch_ti<_Float16>(a, stream);
    return launch_ti<float>(a, stream);
}

}  // namespace wkv7
