// Device helpers shared by the kernels: FP32 and bf16 MFMA tiles, lane
// exchanges in registers (DPP, gfx950 row swaps), and raw staging of
// 8-element input groups.
#pragma once

#include "wkv7_device.h"

namespace wkv7 {

// D += A B on v_mfma_f32_16x16x4_f32. Lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; D[4 (l / 16) + r][l % 16] comes back in element r. The
// output layout is the B-operand layout of the next product.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 MFMA with fp32 accumulation. The 16x16 tiles keep the fp32 layouts
// above: lane l supplies row l % 16 of A and column l % 16 of B, and the
// contraction elements of lane group g = l / 16 are its 8 consecutive vector
// elements; D[4 g + r][l % 16] comes back in
// element r. Only the pairing of a lane's element e in A with the same
// lane group's element e in B matters, so each caller chooses which logical
// contraction index element e stands for, the same way on both sides.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// four words at an 8-byte (not 16-byte) aligned LDS address
typedef uint32_t u32x4a8_t __attribute__((ext_vector_type(4), aligned(8)));

__device__ __forceinline__ f32x4 mfma_bf16_k32(u32x4_t a, u32x4_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ u32x4_t cat(u32x2_t a, u32x2_t b) { return u32x4_t{a.x, a.y, b.x, b.y}; }

// Two fp32 values to one word of two bf16 (lo in bits 0-15), each rounded to
// nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Three-piece bf16 split of two fp32 values, x = h + m + l: each piece is the
// previous remainder rounded to bf16 and each remainder is exact in fp32, so
// the pieces carry 24 significant bits (|x - h - m - l| <= 2^-24 |x|). The
// products h_a h_b + h_a m_b + m_a h_b + h_a l_b + m_a m_b + l_a h_b then
// reproduce an fp32 product up to terms of order 2^-24 |a b| (for |x| above
// about 2^-110, where the last piece is still a normal number).
__device__ __forceinline__ void split3(float x0, float x1, uint32_t &h, uint32_t &m, uint32_t &l) {
    h = pk_bf16(x0, x1);
    x0 -= bf_lo(h);
    x1 -= bf_hi(h);
    m = pk_bf16(x0, x1);
    x0 -= bf_lo(m);
    x1 -= bf_hi(m);
    l = pk_bf16(x0, x1);
}

// Two-piece bf16 split of two fp32 values, x = h + l: h is x rounded to bf16,
// l the remainder rounded to bf16, so |x - h - l| <= 2^-18 |x|. The products
// h_a h_b + h_a l_b + l_a h_b then reproduce a b to about 2^-16 |a b|.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &h, uint32_t &l) {
    h = pk_bf16(x0, x1);
    l = pk_bf16(x0 - bf_lo(h), x1 - bf_hi(h));
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

// Lane exchanges without the LDS crossbar: DPP moves within rows of 16 lanes
// (fused into the adds that use them) and the gfx950 row swaps. swap16(A, B)
// exchanges the odd 16-lane rows of A with the even rows of B: afterwards A
// holds (A row 0, B row 0, A row 2, B row 2) and B (A row 1, B row 1, A row 3,
// B row 3). swap32(A, B) exchanges the upper 32 lanes of A with the lower 32
// of B: afterwards A holds (A low, B low) and B (A high, B high).
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __builtin_amdgcn_update_dpp(0.f, x, CTRL, 0xf, 0xf, false);
}
constexpr int kDppRowRor8 = 0x128, kDppHalfMirror = 0x141, kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E;
__device__ __forceinline__ void swap16(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// Sum over the 16 lanes of a row, in every lane: pairs 8 apart, then the
// mirror within 8, then the quads' two exchanges.
__device__ __forceinline__ float sum16(float k) {
    k += dpp<kDppRowRor8>(k);
    k += dpp<kDppHalfMirror>(k);
    k += dpp<kDppQuadXor1>(k);
    k += dpp<kDppQuadXor2>(k);
    return k;
}
// x[q] summed over the four 16-lane rows of the wave: on return lane row q
// holds the total of x[q] (a reduce-scatter; 2 + 1 swaps).
__device__ __forceinline__ float sum_rows_scatter(const float (&x)[4]) {
    float a0 = x[0], a1 = x[1], a2 = x[2], a3 = x[3];
    swap16(a0, a1);
    swap16(a2, a3);
    float y01 = a0 + a1, y23 = a2 + a3;          // rows 0, 2: x0, x2 over rows (0,1)/(2,3); rows 1, 3: x1, x3
    swap32(y01, y23);
    return y01 + y23;                            // lower half: x0 (row 0), x1 (row 1); upper: x2, x3
}
// The same totals in every lane (3 more swaps).
__device__ __forceinline__ void sum_rows_all(float (&x)[4]) {
    float z = sum_rows_scatter(x), zl = z, zh = z;
    swap32(zl, zh);                              // zl: row q & 1's total, zh: row 2 + (q & 1)'s
    float e0 = zl, o0 = zl, e1 = zh, o1 = zh;
    swap16(e0, o0);                              // e0: row 0's total, o0: row 1's
    swap16(e1, o1);                              // e1: row 2's, o1: row 3's
    x[0] = e0; x[1] = o0; x[2] = e1; x[3] = o1;
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
