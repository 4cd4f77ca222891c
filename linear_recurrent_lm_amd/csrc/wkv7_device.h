// Device-side helpers shared by the WKV-7 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kN = 64;       // head size
constexpr int kChunk = 16;   // checkpoint interval in tokens
// Gated DeltaNet q and k are normalised as x / max(||x||_2, kGdnNormEps).
constexpr float kGdnNormEps = 1e-12f;

// Unit resolution: one (sequence, head) pair. Dense mode: sequence = row.
struct SegParams {
    int32_t B, T, H;
    int32_t num_seqs;            // 0 = dense
    const int32_t *seq_start;
    const int32_t *seq_len;
    const int32_t *seq_ckpt;
    int32_t ckpt_slots;
    int32_t need_ckpt;           // 1 when checkpoints are read or written
};

struct Unit {
    int64_t start;   // flat token index of the first token
    int32_t len;     // 0 = skip
    int64_t ckpt;    // first checkpoint slot
};

// Reads the segment table entry of sequence s and rejects entries that would
// leave the buffers (negative length, crossing a row, checkpoint slots out of
// range): such a sequence is treated as empty.
// Row blocks per unit for the chunked sequential kernels (forward, backward
// sweep): 1 (64-row workgroups), 2 (32 rows) or 4 (16 rows). One workgroup
// fits on a CU (LDS), so a launch of more than 256 workgroups runs in rounds;
// the choice minimises rounds x the time of one chunk step of the shape,
// measured on MI355X at about 5.5K, 4.5K and 3.6K cycles (relative 11:9:7).
inline int row_blocks_for(int64_t units) {
    const int64_t u8 = (units + 7) / 8 * 8;
    const int64_t c1 = (units + 255) / 256 * 11, c2 = (2 * u8 + 255) / 256 * 9, c4 = (4 * u8 + 255) / 256 * 7;
    if (c1 <= c2 && c1 <= c4) return 1;
    return c2 <= c4 ? 2 : 4;
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// only, so global loads issued ahead (prefetch) and global stores stay in
// flight across it. (__syncthreads also waits for every outstanding global
// access of the wave.) The "memory" clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ inline Unit resolve_unit(const SegParams &p, int s) {
    Unit u;
    const int64_t nc = (p.T + kChunk - 1) / kChunk;
    if (p.num_seqs == 0) {
        u.start = (int64_t)s * p.T;
        u.len = p.T;
        u.ckpt = (int64_t)s * nc;
        return u;
    }
    const int64_t st = p.seq_start[s];
    const int64_t ln = p.seq_len[s];
    u.start = st;
    u.len = (int32_t)ln;
    u.ckpt = p.seq_ckpt ? (int64_t)p.seq_ckpt[s] : 0;
    const int64_t total = (int64_t)p.B * p.T;
    bool ok = ln >= 0 && st >= 0 && st + ln <= total;
    if (ok && ln > 0) ok = (st / p.T) == ((st + ln - 1) / p.T);
    if (ok && p.need_ckpt && ln > 0) {
        const int64_t chunks = (ln + kChunk - 1) / kChunk;
        ok = p.seq_ckpt != nullptr && u.ckpt >= 0 && u.ckpt + chunks <= p.ckpt_slots;
    }
    if (!ok) u.len = 0;
    return u;
}

// Offset t * ts + c of token t of a chunk (t < 16) in a [.., T, H, 64]
// stream with row pitch ts = H * 64, in 32 bits: the API bounds H by 2^16,
// so ts < 2^24 and one 24-bit multiply suffices (a 64-bit product per lane
// takes three quarter-rate instructions). The chunk's own 64-bit offset is
// added separately, from uniform values.
__device__ __forceinline__ int32_t row_off(int t, int64_t ts, int c) {
    return (int32_t)__umul24((unsigned)t, (unsigned)ts) + c;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950); NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <typename TI> struct IO;

template <> struct IO<float> {
    __device__ static __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
    __device__ static __forceinline__ void st(float *p, int64_t i, float x) { p[i] = x; }
};

template <> struct IO<uint16_t> {
    __device__ static __forceinline__ float ld(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ static __forceinline__ void st(uint16_t *p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

template <> struct IO<_Float16> {
    __device__ static __forceinline__ float ld(const _Float16 *p, int64_t i) { return (float)p[i]; }
    // fp32 -> fp16 conversion rounds to nearest even
    __device__ static __forceinline__ void st(_Float16 *p, int64_t i, float x) { p[i] = (_Float16)x; }
};

// The decays n w-stream elements stand for: the values themselves, or their
// exponentials when the stream holds log(decay). One uniform branch around
// the whole group keeps the exponentials off the multiplicative path (a
// per-element select would evaluate them anyway).
template <int n>
__device__ __forceinline__ void decay_of(float *x, int logw) {
    if (logw) {
#pragma unroll
        for (int e = 0; e < n; ++e) x[e] = expf(x[e]);
    }
}

// Is flat token `tok` of a row-major [B*T] token space covered by a sequence?
// Binary search over the (sorted) starts; used only to zero uncovered tokens.
__device__ inline bool token_covered(const SegParams &p, int64_t tok) {
    int lo = 0, hi = p.num_seqs - 1, found = -1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)p.seq_start[mid] <= tok) { found = mid; lo = mid + 1; }
        else hi = mid - 1;
    }
    if (found < 0) return false;
    return tok < (int64_t)p.seq_start[found] + (int64_t)p.seq_len[found];
}

}  // namespace wkv7
