// Launch interfaces of the vocabulary cross-entropy kernels (host side, C++).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vce {

// Macro tile of the bf16 MFMA GEMM: BI rows of A (vocabulary rows in the
// logit tiles) by BJ rows of B (token rows), BK along the contraction per
// pipeline stage. Token rows are padded to a multiple of kBJ, vocabulary
// rows (and a chunk of them) to a multiple of kBI.
constexpr int kBI = 256;
constexpr int kBJ = 256;
constexpr int kBK = 64;

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Largest grid (workgroups) a launch may take: 2^22 workgroups of at most 512
// threads keep every launch below 2^31 threads.
constexpr int64_t kMaxBlocks = (int64_t)1 << 22;

// Forward split of the vocabulary: enough workgroups to fill the chip.
struct FwdPlan {
    int n_itiles, n_jtiles, nsplit, tiles_per_split;
};
FwdPlan fwd_plan(int M, int V);

struct FwdArgs {
    int M, D, V;
    const uint16_t *h, *w;           // bf16 bits, [M, D] and [V, D]
    const int32_t *targets;          // [M]
    float *loss, *lse;               // [M]
    float2 *part;                    // [nsplit, M] running (max, sum), base-2 units
    float *zt;                       // [M] target logit
};
hipError_t launch_forward(const FwdArgs &a, hipStream_t stream);

struct BwdArgs {
    int M, D, V, Vc;                 // Vc: vocabulary rows per chunk
    const uint16_t *h, *w;
    const int32_t *targets;
    const float *lse, *dloss;
    float *dh, *dw;
    uint16_t *wt, *ht, *g, *gt;      // workspace: W^T [D, Vp], h^T [D, Mp], G [Mp, Vcp], G^T [Vcp, Mp]
};
hipError_t launch_backward(const BwdArgs &a, hipStream_t stream);

}  // namespace vce
