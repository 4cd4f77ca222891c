// Issue-pipe probe for gfx950: does a wave's VALU work progress while another
// wave on the same SIMD issues matrix (MFMA) instructions?
//
// One 512-thread workgroup per CU, eight waves, so each SIMD holds two of
// them (wave w and wave w + 4; every wave records its hardware SIMD id so the
// pairing can be checked). Waves 0-3 run `mfma_iters` iterations of four
// independent MFMA accumulator chains, waves 4-7 run `valu_iters` iterations
// of eight independent fp32 FMA chains; either side can be switched off. Each
// wave records the shader-clock cycles of its own loop (its results are
// consumed before the second clock read). Comparing both-on against each
// side alone shows whether the two kinds of work overlap on one SIMD
// (both-on ~ max of the two) or share one issue pipe (both-on ~ their sum).
//
// Built into its own library (libwkv7_probe.so), used only by the
// measurement script; the WKV-7 library does not contain it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t cycles_now() {
    int64_t t;
    asm volatile("s_memtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
    return t;
}

__device__ __forceinline__ int64_t realtime_now() {
    int64_t t;
    asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t)::"memory");
    return t;
}

__device__ __forceinline__ void consume(float x) { asm volatile("; consume %0" ::"v"(x) : "memory"); }

// kind 0: v_mfma_f32_16x16x4_f32; 1: v_mfma_f32_32x32x2_f32;
// 2: v_mfma_f32_16x16x32_bf16; 4: v_mfma_f32_16x16x16_bf16;
// 5: v_mfma_f32_16x16x32_bf16 with eight accumulator chains;
// 6: v_mfma_f32_16x16x32_bf16, one chain; 7: v_mfma_f32_16x16x4_f32, one chain.
template <int KIND>
__device__ float mfma_loop(int iters, float x) {
    if constexpr (KIND == 0) {
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, x, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, x, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, x, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, x, c3, 0, 0, 0);
        }
        return c0[0] + c1[1] + c2[2] + c3[3];
    } else if constexpr (KIND == 1) {
        f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, x, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, x, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, x, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, x, c3, 0, 0, 0);
        }
        return c0[0] + c1[1] + c2[2] + c3[3];
    } else if constexpr (KIND == 4) {
        i16x4 a;
        for (int e = 0; e < 4; ++e) a[e] = (short)(__builtin_bit_cast(unsigned, x + 0.125f * e) >> 16);
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, a, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, a, c3, 0, 0, 0);
        }
        return c0[0] + c1[1] + c2[2] + c3[3];
    } else if constexpr (KIND == 6) {
        bf16x8 a;
        for (int e = 0; e < 8; ++e) a[e] = (__bf16)(x + 0.125f * e);
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c0, 0, 0, 0);
        }
        return c0[0] + c0[3];
    } else if constexpr (KIND == 7) {
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x, x, c0, 0, 0, 0);
        }
        return c0[0] + c0[3];
    } else if constexpr (KIND == 5) {
        bf16x8 a;
        for (int e = 0; e < 8; ++e) a[e] = (__bf16)(x + 0.125f * e);
        f32x4 c[8];
        for (int q = 0; q < 8; ++q) c[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < iters; i += 2) {
#pragma unroll
            for (int q = 0; q < 8; ++q) c[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c[q], 0, 0, 0);
        }
        return c[0][0] + c[1][1] + c[2][2] + c[3][3] + c[4][0] + c[5][1] + c[6][2] + c[7][3];
    } else {
        bf16x8 a;
        for (int e = 0; e < 8; ++e) a[e] = (__bf16)(x + 0.125f * e);
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
        for (int i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c3, 0, 0, 0);
        }
        return c0[0] + c1[1] + c2[2] + c3[3];
    }
}

// m, c: multiplier and addend from kernel arguments (scalar registers, so
// every FMA is a plain 32-bit-encoded v_fma_f32 with no literal).
__device__ float valu_loop(int iters, float x, float m, float c) {
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = x + (float)e;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = fmaf(a[e], m, c);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += a[e];
    return s;
}

// rec[(block * 8 + wave) * 4 + 0] = loop cycles (s_memtime), [+1] = loop
// ticks of the constant-rate s_memrealtime counter, [+2] = HW_ID register.
// KIND 3: waves 0-3 run the VALU loop as well (two VALU waves per SIMD).
template <int KIND>
__global__ __launch_bounds__(512) void pipe_probe_kernel(int side_mask, int mfma_iters, int valu_iters,
                                                         float m, float c, int64_t *rec, float *sink) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float x = 1e-3f * (float)lane;
    // HW_ID (hwreg 4), all 32 bits: SIMD id in bits 5:4
    const int hwid = __builtin_amdgcn_s_getreg((31 << 11) | 4);
    __syncthreads();
    int64_t t0 = 0, t1 = 0, r0 = 0, r1 = 0;
    float s = 0.f;
    if (wave < 4 && (side_mask & 1)) {
        r0 = realtime_now();
        t0 = cycles_now();
        if constexpr (KIND == 3)
            s = valu_loop(mfma_iters, x, m, c);
        else
            s = mfma_loop<KIND>(mfma_iters, x);
        consume(s);
        t1 = cycles_now();
        r1 = realtime_now();
    } else if (wave >= 4 && (side_mask & 2)) {
        r0 = realtime_now();
        t0 = cycles_now();
        s = valu_loop(valu_iters, x, m, c);
        consume(s);
        t1 = cycles_now();
        r1 = realtime_now();
    }
    if (lane == 0) {
        int64_t *o = rec + (blockIdx.x * 8 + wave) * 4;
        o[0] = t1 - t0;
        o[1] = r1 - r0;
        o[2] = hwid;
        o[3] = 0;
    }
    sink[blockIdx.x * 512 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Runs the probe on `blocks` workgroups (rec: device int64 [blocks * 32],
// sink: device float [blocks * 512]). kind: 0 = fp32 16x16x4, 1 = fp32
// 32x32x2, 2 = bf16 16x16x32 MFMA, 3 = VALU on waves 0-3 as well,
// 4 = bf16 16x16x16, 5 = bf16 16x16x32 on eight chains, 6 = bf16 16x16x32
// on one chain, 7 = fp32 16x16x4 on one chain;
// side_mask: 1 = waves 0-3 on, 2 = waves 4-7 on. Returns 0 on success,
// else the HIP error code.
int wkv7_probe_pipe(int kind, int side_mask, int mfma_iters, int valu_iters, int blocks, int64_t *rec,
                    float *sink, void *stream) {
    if (blocks < 1 || mfma_iters < 0 || valu_iters < 0 || !rec || !sink) return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    const float m = 0.999f, c = 1e-3f;
    switch (kind) {
    case 0:
        hipLaunchKernelGGL(pipe_probe_kernel<0>, dim3(blocks), dim3(512), 0, s, side_mask, mfma_iters, valu_iters, m, c, rec, sink);
        break;
    case 1:
        hipLaunchKernelGGL(pipe_probe_kernel<1>, dim3(blocks), dim3(512), 0, s, side_mask, mfma_iters, valu_iters, m, c, rec, sink);
        break;
    case 2:
        hipLaunchKernelGGL(pipe_probe_kernel<2>, dim3(blocks), dim3(512), 0, s, side_mask, mfma_iters, valu_iters, m, c, rec, sink);
        break;
    case 3:
        hipLaunchKernelGGL(pipe_probe_kernel<3>, dim3(blocks), dim3(512), 0, s, side_mask, mfma_iters, valu_iters, m, c, rec, sink);
        break;
    case 4:
        hipLaunchKernelGGL(pipe_probe_kernel<4>, dim3(blocks), dim3(512), 0, s, side_mask, mfma_iters, valu_iters, m, c, rec, sink);
        break;
    case 5:
        hipLaunchKernelGGL(pipe_probe_kernel<5>, dim3(blocks), dim3(512), 0, s, side_mask, mfma_iters, valu_iters, m, c, rec, sink);
        break;
    case 6:
        hipLaunchKernelGGL(pipe_probe_kernel<6>, dim3(blocks), dim3(512), 0, s, side_mask, mfma_iters, valu_iters, m, c, rec, sink);
        break;
    case 7:
        hipLaunchKernelGGL(pipe_probe_kernel<7>, dim3(blocks), dim3(512), 0, s, side_mask, mfma_iters, valu_iters, m, c, rec, sink);
        break;
    default:
        return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
