// Device helpers shared by the chunk kernels: FP32 MFMA tiles, DPP lane
// permutations within quads, and raw staging of 8-element input groups.
#pragma once

#include "wkv7_device.h"

namespace wkv7 {

// D += A B on v_mfma_f32_16x16x4_f32. Lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; D[4 (l / 16) + r][l % 16] comes back in element r. The
// output layout is the B-operand layout of the next product.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16x16 product over K = 64: D[m][n] = sum_j A_m[j] B_n[j], where this lane
// supplies row m = lane % 16 of A (arow) and row n = lane % 16 of B (brow),
// both 16-byte aligned rows of 64 floats.
__device__ __forceinline__ f32x4 rows_product(const float *arow, const float *brow, int kq) {
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const float4 a = *(const float4 *)(arow + 16 * g + 4 * kq);
        const float4 b = *(const float4 *)(brow + 16 * g + 4 * kq);
        d = mfma4(a.x, b.x, d); d = mfma4(a.y, b.y, d);
        d = mfma4(a.z, b.z, d); d = mfma4(a.w, b.w, d);
    }
    return d;
}

// Lane permutations within groups of 4 lanes (DPP quad_perm).
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float quad_bcast(float v, int k) {   // value of quad lane k
    switch (k) {
    case 0: return quad_perm<0x00>(v);
    case 1: return quad_perm<0x55>(v);
    case 2: return quad_perm<0xaa>(v);
    default: return quad_perm<0xff>(v);
    }
}
__device__ __forceinline__ float quad_sum(float v) {
    v += quad_perm<0xb1>(v);      // lanes ^1
    v += quad_perm<0x4e>(v);      // lanes ^2
    return v;
}

// Raw input data in flight: K groups of 8 elements per staging thread, kept
// packed until use so that the loads are not consumed early.
template <typename TI, int K> struct Raw;
template <int K> struct Raw<uint16_t, K> { uint4 q[K]; };
template <int K> struct Raw<float, K> { float4 q[K][2]; };
template <int K> struct Raw<_Float16, K> { uint4 q[K]; };

template <int K>
__device__ __forceinline__ void raw_load(const uint16_t *p, Raw<uint16_t, K> &r, int k) {
    r.q[k] = *(const uint4 *)p;
}
template <int K>
__device__ __forceinline__ void raw_load(const float *p, Raw<float, K> &r, int k) {
    r.q[k][0] = *(const float4 *)p;
    r.q[k][1] = *(const float4 *)(p + 4);
}
template <int K>
__device__ __forceinline__ void raw_unpack(const Raw<uint16_t, K> &r, int k, float *x) {
    const uint32_t u[4] = {r.q[k].x, r.q[k].y, r.q[k].z, r.q[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(u[e] << 16);
        x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
}
template <int K>
__device__ __forceinline__ void raw_load(const _Float16 *p, Raw<_Float16, K> &r, int k) {
    r.q[k] = *(const uint4 *)p;
}
__device__ __forceinline__ float half_lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}
template <int K>
__device__ __forceinline__ void raw_unpack(const Raw<_Float16, K> &r, int k, float *x) {
    const uint32_t u[4] = {r.q[k].x, r.q[k].y, r.q[k].z, r.q[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = half_lo(u[e]);
        x[2 * e + 1] = half_hi(u[e]);
    }
}
template <int K>
__device__ __forceinline__ void raw_unpack(const Raw<float, K> &r, int k, float *x) {
    x[0] = r.q[k][0].x; x[1] = r.q[k][0].y; x[2] = r.q[k][0].z; x[3] = r.q[k][0].w;
    x[4] = r.q[k][1].x; x[5] = r.q[k][1].y; x[6] = r.q[k][1].z; x[7] = r.q[k][1].w;
}

// Four consecutive input elements (one 8- or 16-byte load) per staging group.
template <typename TI> struct Raw4;
template <> struct Raw4<uint16_t> { uint2 q; };
template <> struct Raw4<float> { float4 q; };
template <> struct Raw4<_Float16> { uint2 q; };
__device__ __forceinline__ void raw4_load(const uint16_t *p, Raw4<uint16_t> &r) { r.q = *(const uint2 *)p; }
__device__ __forceinline__ void raw4_load(const float *p, Raw4<float> &r) { r.q = *(const float4 *)p; }
__device__ __forceinline__ void raw4_unpack(const Raw4<uint16_t> &r, float *x) {
    x[0] = __uint_as_float(r.q.x << 16); x[1] = __uint_as_float(r.q.x & 0xffff0000u);
    x[2] = __uint_as_float(r.q.y << 16); x[3] = __uint_as_float(r.q.y & 0xffff0000u);
}
__device__ __forceinline__ void raw4_load(const _Float16 *p, Raw4<_Float16> &r) { r.q = *(const uint2 *)p; }
__device__ __forceinline__ void raw4_unpack(const Raw4<_Float16> &r, float *x) {
    x[0] = half_lo(r.q.x); x[1] = half_hi(r.q.x); x[2] = half_lo(r.q.y); x[3] = half_hi(r.q.y);
}
__device__ __forceinline__ void raw4_unpack(const Raw4<float> &r, float *x) {
    x[0] = r.q.x; x[1] = r.q.y; x[2] = r.q.z; x[3] = r.q.w;
}

}  // namespace wkv7
