// Segment mode: tokens that no sequence covers get zeros in the given
// output streams (y in the forward, the six gradients in the backward), so
// outputs at padding are defined without ever reading the padding's inputs.
#include "wkv7_kernels.h"

namespace wkv7 {
namespace {

struct PtrPack {
    void *p[6];
};

template <typename TI>
__global__ __launch_bounds__(256) void zero_uncovered_kernel(SegParams seg, PtrPack ptrs, int nptr) {
    // One thread per (flat token, head): 64 contiguous elements per stream.
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ntok = (int64_t)seg.B * seg.T;
    if (idx >= ntok * seg.H) return;
    const int64_t tok = idx / seg.H;
    if (token_covered(seg, tok)) return;
    for (int q = 0; q < nptr; ++q) {
        TI *dst = (TI *)ptrs.p[q] + idx * kN;
#pragma unroll
        for (int e = 0; e < kN; ++e) dst[e] = TI(0);
    }
}

}  // namespace

hipError_t launch_zero_uncovered(const SegParams &seg, int dtype, void *const *ptrs, int nptr,
                                 hipStream_t stream) {
    PtrPack pk{};
    for (int q = 0; q < nptr && q < 6; ++q) pk.p[q] = ptrs[q];
    const int64_t n = (int64_t)seg.B * seg.T * seg.H;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dtype != 0)            // bf16 and fp16: 2-byte zeros
        hipLaunchKernelGGL(zero_uncovered_kernel<uint16_t>, grid, dim3(256), 0, stream, seg, pk, nptr);
    else
        hipLaunchKernelGGL(zero_uncovered_kernel<float>, grid, dim3(256), 0, stream, seg, pk, nptr);
    return hipGetLastError();
}

}  // namespace wkv7
