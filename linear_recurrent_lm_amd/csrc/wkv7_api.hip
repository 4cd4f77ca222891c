// Host side of libwkv7.so: the C ABI declared in include/wkv7.h.
// Every argument is checked before anything touches the HIP runtime, so the
// validation paths work (and are tested) on machines without a GPU.
#include <cmath>
#include <atomic>
#include <cstring>

#include <hip/hip_runtime.h>

#include "../../include/vocab_ce.h"
#include "../../include/wkv7.h"
#include "vce_kernels.h"
#include "wkv7_kernels.h"

namespace {

using wkv7::kChunk;
using wkv7::kN;

constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr int32_t kMaxHeads = 1 << 16;      // keeps a stream's row pitch H * 64 below 2^24

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

size_t elem_size(int dtype) { return dtype == WKV7_F32 ? 4 : 2; }

// A buffer as a byte range; a null pointer or zero size takes no part in the
// overlap checks.
struct Range {
    const void *p;
    size_t n;
};

// Does any output range overlap an input range or another output range?
// Outputs are written while inputs are still read (and by other lanes of the
// same kernels), so no output may share a byte with any other buffer.
bool any_overlap(const Range *ins, int nin, const Range *outs, int nout) {
    for (int o = 0; o < nout; ++o) {
        if (!outs[o].p || !outs[o].n) continue;
        for (int q = 0; q < nin; ++q)
            if (ins[q].p && ins[q].n && ranges_overlap(ins[q].p, ins[q].n, outs[o].p, outs[o].n)) return true;
        for (int o2 = o + 1; o2 < nout; ++o2)
            if (outs[o2].p && outs[o2].n && ranges_overlap(outs[o].p, outs[o].n, outs[o2].p, outs[o2].n))
                return true;
    }
    return false;
}

bool dtype_ok(int32_t dtype) { return dtype == WKV7_F32 || dtype == WKV7_BF16 || dtype == WKV7_F16; }

// wide: the call also takes head size 128 (the forward, the backward and its
// workspace query do; the allocation-free backward does not).
wkv7_status check_desc(const wkv7_desc *d, bool wide = false) {
    if (!d) return WKV7_ERR_INVALID_ARGUMENT;
    if (d->N != kN && !(wide && d->N == 128)) return WKV7_ERR_UNSUPPORTED;
    if (!dtype_ok(d->dtype)) return WKV7_ERR_UNSUPPORTED;
    if (d->decay != WKV7_DECAY_MULT && d->decay != WKV7_DECAY_LOG) return WKV7_ERR_UNSUPPORTED;
    if (d->grad_f32 != 0 && d->grad_f32 != 1) return WKV7_ERR_INVALID_ARGUMENT;
    if (d->B < 1 || d->T < 1 || d->H < 1 || d->H > kMaxHeads) return WKV7_ERR_INVALID_ARGUMENT;
    const int64_t toks = (int64_t)d->B * d->T;
    if (toks > INT32_MAX) return WKV7_ERR_INVALID_ARGUMENT;
    if (toks * d->H * d->N > kMaxElems) return WKV7_ERR_INVALID_ARGUMENT;
    if (d->num_seqs < 0) return WKV7_ERR_INVALID_ARGUMENT;
    if (d->num_seqs > 0 && (!d->seq_start || !d->seq_len)) return WKV7_ERR_INVALID_ARGUMENT;
    const int64_t S = d->num_seqs > 0 ? d->num_seqs : d->B;
    if (S * d->H > INT32_MAX) return WKV7_ERR_INVALID_ARGUMENT;
    return WKV7_OK;
}

int64_t num_states(const wkv7_desc *d) { return d->num_seqs > 0 ? d->num_seqs : d->B; }

// Bytes of one [B, T, H, N] token stream with elements of `dtype`.
size_t stream_bytes(const wkv7_desc *d, int32_t dtype) {
    return (size_t)d->B * d->T * d->H * d->N * elem_size(dtype);
}

// Bytes of the checkpoint buffer the descriptor implies.
size_t ckpt_bytes(const wkv7_desc *d) {
    const int64_t slots = d->num_seqs > 0 ? (d->ckpt_slots > 0 ? d->ckpt_slots : 0)
                                          : (int64_t)d->B * ((d->T + kChunk - 1) / kChunk);
    return (size_t)slots * d->H * d->N * d->N * sizeof(float);
}

wkv7_status check_streams(const void *const *ptrs, int n) {
    for (int q = 0; q < n; ++q)
        if (!ptrs[q] || !aligned16(ptrs[q])) return WKV7_ERR_INVALID_ARGUMENT;
    return WKV7_OK;
}

wkv7_status check_ckpt(const wkv7_desc *d, const float *ckpt) {
    if (!ckpt) return WKV7_OK;
    if (!aligned16(ckpt)) return WKV7_ERR_INVALID_ARGUMENT;
    if (d->num_seqs > 0 && (!d->seq_ckpt || d->ckpt_slots < 0)) return WKV7_ERR_INVALID_ARGUMENT;
    return WKV7_OK;
}

// 0 = unknown, 1 = gfx950, 2 = other / unusable.
std::atomic<int> g_dev_ok[64];

wkv7_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return WKV7_ERR_HIP;
    if (dev < 0 || dev >= 64) return WKV7_ERR_UNSUPPORTED;
    int st = g_dev_ok[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return WKV7_ERR_HIP;
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_ok[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? WKV7_OK : WKV7_ERR_UNSUPPORTED;
}

wkv7::SegParams seg_params(const wkv7_desc *d, bool need_ckpt) {
    wkv7::SegParams s;
    s.B = d->B; s.T = d->T; s.H = d->H;
    s.num_seqs = d->num_seqs;
    s.seq_start = d->seq_start;
    s.seq_len = d->seq_len;
    s.seq_ckpt = d->seq_ckpt;
    s.ckpt_slots = d->ckpt_slots;
    s.need_ckpt = need_ckpt ? 1 : 0;
    return s;
}


// Vocabulary cross-entropy: size limits and workspace layout.
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

size_t pad256(size_t x) { return (x + 255) / 256 * 256; }

wkv7_status vce_check_sizes(int32_t M, int32_t D, int32_t V) {
    if (M < 1 || M > (1 << 28)) return WKV7_ERR_INVALID_ARGUMENT;
    if (D < 64 || D > 65536 || D % 64 != 0) return WKV7_ERR_INVALID_ARGUMENT;
    if (V < 1 || V > (1 << 24)) return WKV7_ERR_INVALID_ARGUMENT;
    const vce::FwdPlan f = vce::fwd_plan(M, V);
    if ((int64_t)f.n_jtiles * f.nsplit > vce::kMaxBlocks) return WKV7_ERR_INVALID_ARGUMENT;
    return WKV7_OK;
}

struct VceBwdLayout {
    int32_t Vc;
    size_t wt, ht, g, gt, total;     // byte offsets
};

// [W^T: D x Vp][h^T: D x Mp][G: Mp x Vcp][G^T: Vcp x Mp], bf16, each 256-byte aligned.
wkv7_status vce_bwd_layout(int32_t M, int32_t D, int32_t V, int32_t vocab_chunk, VceBwdLayout *l) {
    wkv7_status st = vce_check_sizes(M, D, V);
    if (st != WKV7_OK) return st;
    if (vocab_chunk < 1) return WKV7_ERR_INVALID_ARGUMENT;
    // whole tiles of kBI vocabulary rows per chunk
    const int64_t vc = vce::round_up(vocab_chunk < V ? vocab_chunk : V, vce::kBI);
    l->Vc = (int32_t)(vc < V ? vc : V);
    const int64_t Vp = vce::round_up(V, vce::kBI), Mp = vce::round_up(M, vce::kBJ);
    const int64_t Vcp = vce::round_up(l->Vc, vce::kBI);
    // every launch (workgroups of up to 512 threads) must stay below 2^31 threads
    const int64_t dt = vce::round_up(D, vce::kBJ) / vce::kBJ;
    const int64_t grids[3] = {(Vcp / vce::kBI) * (Mp / vce::kBJ),     // gradient tiles
                              (Mp / vce::kBI) * dt,                   // dh
                              (Vcp / vce::kBI) * dt};                 // dW
    for (int64_t g : grids)
        if (g > vce::kMaxBlocks) return WKV7_ERR_INVALID_ARGUMENT;
    l->wt = 0;
    l->ht = l->wt + pad256((size_t)D * Vp * 2);
    l->g = l->ht + pad256((size_t)D * Mp * 2);
    l->gt = l->g + pad256((size_t)Mp * Vcp * 2);
    l->total = l->gt + pad256((size_t)Vcp * Mp * 2);
    return WKV7_OK;
}

// Segment mode: the backward's list of (sequence, chunk group) work items
// after the per-chunk results: a count and at most ceil(slots / 8) +
// num_seqs int32 pairs (a bound for groups of 8 or more chunks; the kernel's
// groups are 16).
int64_t glist_cap(int64_t slots, int64_t num_seqs) { return (slots + 7) / 8 + num_seqs; }
size_t glist_bytes(int64_t slots, int64_t num_seqs) { return (size_t)(1 + 2 * glist_cap(slots, num_seqs)) * 4; }

size_t vce_fwd_bytes(int32_t M, int32_t V) {
    const vce::FwdPlan f = vce::fwd_plan(M, V);
    return pad256((size_t)f.nsplit * M * 8) + pad256((size_t)M * 4);
}

// Device address of `scratch` (below) on each device, looked up once per
// device on the first wkv7_backward_noalloc call made with it current. In host
// code the array's name is only a stand-in for the symbol, never an address
// a kernel may use.
std::atomic<void *> g_scratch[64];

wkv7_status scratch_address(void **out);

}  // namespace

// Static scratch of wkv7_backward_noalloc: the backward's per-chunk workspace
// for callers that cannot allocate. Each device holds its own copy for the
// life of the process; calls on one device share it.
static __device__ __align__(256) unsigned char scratch[WKV7_STATIC_SCRATCH_BYTES];

namespace {

wkv7_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return WKV7_ERR_HIP;
    if (dev < 0 || dev >= 64) return WKV7_ERR_UNSUPPORTED;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WKV7_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return WKV7_OK;
}

}  // namespace

extern "C" {

int32_t wkv7_abi_version(void) { return WKV7_ABI_VERSION; }

const char *wkv7_status_string(wkv7_status s) {
    switch (s) {
    case WKV7_OK: return "ok";
    case WKV7_ERR_INVALID_ARGUMENT: return "invalid argument";
    case WKV7_ERR_UNSUPPORTED: return "unsupported";
    case WKV7_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case WKV7_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

wkv7_status wkv7_checkpoint_slots(int32_t B, int32_t T, int64_t *slots) {
    if (!slots || B < 1 || T < 1) return WKV7_ERR_INVALID_ARGUMENT;
    *slots = (int64_t)B * ((T + kChunk - 1) / kChunk);
    return WKV7_OK;
}

wkv7_status wkv7_workspace_bytes(const wkv7_desc *d, size_t *bytes) {
    if (!bytes) return WKV7_ERR_INVALID_ARGUMENT;
    const wkv7_status st = check_desc(d, true);
    if (st != WKV7_OK) return st;
    if (d->N == 128) {
        // one workgroup per (sequence, head) sums every gradient itself
        if (d->num_seqs > 0 && d->ckpt_slots < 0) return WKV7_ERR_INVALID_ARGUMENT;
        *bytes = 0;
        return WKV7_OK;
    }
    // per checkpoint slot and head: the fp32 64x64 state gradient leaving the
    // chunk, the fp32 16x64 drhs and the fp32 16x16 W of the chunk
    int64_t slots = 0;
    if (d->num_seqs > 0) {
        if (d->ckpt_slots < 0) return WKV7_ERR_INVALID_ARGUMENT;
        slots = d->ckpt_slots;
    } else {
        slots = (int64_t)d->B * ((d->T + kChunk - 1) / kChunk);
    }
    *bytes = (size_t)slots * d->H * (kN * kN + kChunk * kN + kChunk * kChunk) * sizeof(float);
    if (d->num_seqs > 0) *bytes += pad256(glist_bytes(slots, d->num_seqs));
    return WKV7_OK;
}

wkv7_status wkv7_segments_check(int32_t B, int32_t T, int32_t num_seqs, const int32_t *seq_start,
                                const int32_t *seq_len, int32_t *seq_ckpt_out, int64_t *slots_out) {
    if (B < 1 || T < 1 || num_seqs < 0) return WKV7_ERR_INVALID_ARGUMENT;
    if (num_seqs > 0 && (!seq_start || !seq_len)) return WKV7_ERR_INVALID_ARGUMENT;
    const int64_t total = (int64_t)B * T;
    int64_t prev_end = 0, slots = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t st = seq_start[s], ln = seq_len[s];
        if (ln < 0 || st < 0 || st + ln > total) return WKV7_ERR_INVALID_ARGUMENT;
        if (st < prev_end) return WKV7_ERR_INVALID_ARGUMENT;   // unsorted or overlapping
        if (ln > 0 && st / T != (st + ln - 1) / T) return WKV7_ERR_INVALID_ARGUMENT;
        prev_end = st + ln;
        if (slots > INT32_MAX) return WKV7_ERR_INVALID_ARGUMENT;
        if (seq_ckpt_out) seq_ckpt_out[s] = (int32_t)slots;
        slots += (ln + kChunk - 1) / kChunk;
    }
    if (slots > INT32_MAX) return WKV7_ERR_INVALID_ARGUMENT;
    if (slots_out) *slots_out = slots;
    return WKV7_OK;
}

wkv7_status wkv7_forward(const wkv7_desc *d, const void *r, const void *w, const void *k,
                         const void *v, const void *a, const void *b, const float *s0, void *y,
                         float *s_out, float *ckpt, void *stream) {
    wkv7_status st = check_desc(d, true);
    if (st != WKV7_OK) return st;
    const void *streams[7] = {r, w, k, v, a, b, y};
    if ((st = check_streams(streams, 7)) != WKV7_OK) return st;
    if ((s0 && !aligned16(s0)) || (s_out && !aligned16(s_out))) return WKV7_ERR_INVALID_ARGUMENT;
    if ((st = check_ckpt(d, ckpt)) != WKV7_OK) return st;
    {
        const size_t state_bytes = (size_t)num_states(d) * d->H * d->N * d->N * sizeof(float);
        const size_t sb = stream_bytes(d, d->dtype);
        const Range ins[7] = {{r, sb}, {w, sb}, {k, sb}, {v, sb}, {a, sb}, {b, sb}, {s0, state_bytes}};
        const Range outs[3] = {{y, sb}, {s_out, state_bytes}, {ckpt, ckpt_bytes(d)}};
        if (any_overlap(ins, 7, outs, 3)) return WKV7_ERR_INVALID_ARGUMENT;
    }
    if ((st = check_device()) != WKV7_OK) return st;

    hipStream_t hs = (hipStream_t)stream;
    wkv7::FwdArgs args;
    args.seg = seg_params(d, ckpt != nullptr);
    args.dtype = d->dtype;
    args.logw = d->decay == WKV7_DECAY_LOG;
    args.r = r; args.w = w; args.k = k; args.v = v; args.a = a; args.b = b;
    args.s0 = s0; args.y = y; args.s_out = s_out; args.ckpt = ckpt;
    if (d->num_seqs > 0) {
        // a [.., H, 128] stream is laid out as [.., 2H, 64]
        wkv7::SegParams zs = args.seg;
        zs.H = d->H * (d->N / kN);
        void *outs[1] = {y};
        if (wkv7::launch_zero_uncovered(zs, d->dtype, outs, 1, hs) != hipSuccess)
            return WKV7_ERR_HIP;
    }
    // head size 128: the lean chunk form; head size 64: the warp-specialised
    // chunk form
    hipError_t e;
    if (d->N == 128)
        e = wkv7::launch_forward_cf(args, 128, hs);
    else
        e = wkv7::launch_forward(args, hs);
    if (e != hipSuccess) return WKV7_ERR_HIP;
    return WKV7_OK;
}

// The backward with the caller's workspace, or (use_scratch) with the
// library's static scratch of this device in its place.
static wkv7_status backward_impl(const wkv7_desc *d, const void *r, const void *w, const void *k,
                                 const void *v, const void *a, const void *b, const float *ckpt,
                                 const void *dy, const float *ds_out, void *dr, void *dw, void *dk,
                                 void *dv, void *da, void *db, float *ds0, void *workspace,
                                 size_t workspace_bytes, bool use_scratch, void *stream) {
    wkv7_status st = check_desc(d, !use_scratch);
    if (st != WKV7_OK) return st;
    const bool wide = d->N == 128;
    const void *streams[12] = {r, w, k, v, a, b, dr, dw, dk, dv, da, db};
    if ((st = check_streams(streams, 12)) != WKV7_OK) return st;
    if (dy && !aligned16(dy)) return WKV7_ERR_INVALID_ARGUMENT;
    if ((ds_out && !aligned16(ds_out)) || (ds0 && !aligned16(ds0))) return WKV7_ERR_INVALID_ARGUMENT;
    if (!ckpt) return WKV7_ERR_INVALID_ARGUMENT;
    if ((st = check_ckpt(d, ckpt)) != WKV7_OK) return st;
    size_t need = 0;
    if ((st = wkv7_workspace_bytes(d, &need)) != WKV7_OK) return st;
    {
        // the second pass's grid: work items x heads (segment mode) or
        // ceil(T / 128) chunk groups x B x H (dense) workgroups; at head
        // size 128, one workgroup per (sequence, head)
        const int64_t items = wide ? num_states(d)
                              : d->num_seqs > 0 ? glist_cap(d->ckpt_slots, d->num_seqs)
                                                : (int64_t)d->B * ((d->T + 127) / 128);
        if (items * d->H > INT32_MAX) return WKV7_ERR_INVALID_ARGUMENT;
    }
    if (use_scratch) {
        if (need > WKV7_STATIC_SCRATCH_BYTES) return WKV7_ERR_WORKSPACE_TOO_SMALL;
    } else {
        if (workspace_bytes < need || (need > 0 && !workspace)) return WKV7_ERR_WORKSPACE_TOO_SMALL;
        if (workspace && !aligned16(workspace)) return WKV7_ERR_INVALID_ARGUMENT;
    }
    {
        const size_t state_bytes = (size_t)num_states(d) * d->H * d->N * d->N * sizeof(float);
        const size_t sb = stream_bytes(d, d->dtype);
        const size_t gb = stream_bytes(d, d->grad_f32 ? WKV7_F32 : d->dtype);
        const Range ins[9] = {{r, sb}, {w, sb}, {k, sb}, {v, sb}, {a, sb}, {b, sb},
                              {ckpt, ckpt_bytes(d)}, {dy, sb}, {ds_out, state_bytes}};
        const Range outs[8] = {{dr, gb}, {dw, gb}, {dk, gb}, {dv, gb}, {da, gb}, {db, gb},
                               {ds0, state_bytes}, {workspace, need}};
        if (any_overlap(ins, 9, outs, 8)) return WKV7_ERR_INVALID_ARGUMENT;
    }
    if ((st = check_device()) != WKV7_OK) return st;
    if (use_scratch && (st = scratch_address(&workspace)) != WKV7_OK) return st;

    hipStream_t hs = (hipStream_t)stream;
    wkv7::BwdArgs args;
    args.seg = seg_params(d, true);
    args.dtype = d->dtype;
    args.logw = d->decay == WKV7_DECAY_LOG;
    args.grad_f32 = d->grad_f32;
    args.r = r; args.w = w; args.k = k; args.v = v; args.a = a; args.b = b;
    args.ckpt = ckpt; args.dy = dy; args.ds_out = ds_out;
    args.dr = dr; args.dw = dw; args.dk = dk; args.dv = dv; args.da = da; args.db = db;
    args.ds0 = ds0;
    args.ws = (float *)workspace;
    if (wide) {
        args.ws_dr = args.ws_w = nullptr;
        args.glist = nullptr;
        args.glist_cap = 0;
        if (d->num_seqs > 0) {
            // a [.., H, 128] stream is laid out as [.., 2H, 64]
            wkv7::SegParams zs = args.seg;
            zs.H = d->H * 2;
            void *outs[6] = {dr, dw, dk, dv, da, db};
            if (wkv7::launch_zero_uncovered(zs, d->grad_f32 ? WKV7_F32 : d->dtype, outs, 6, hs) != hipSuccess)
                return WKV7_ERR_HIP;
        }
        if (wkv7::launch_backward128(args, hs) != hipSuccess) return WKV7_ERR_HIP;
        return WKV7_OK;
    }
    {
        const int64_t slots = d->num_seqs > 0 ? d->ckpt_slots : (int64_t)d->B * ((d->T + kChunk - 1) / kChunk);
        args.ws_dr = args.ws + slots * d->H * kN * kN;
        args.ws_w = args.ws_dr + slots * d->H * kChunk * kN;
        args.glist = nullptr;
        args.glist_cap = 0;
        if (d->num_seqs > 0) {
            // 256-byte aligned start after the fp32 arrays
            const size_t off = (size_t)slots * d->H * (kN * kN + kChunk * kN + kChunk * kChunk) * sizeof(float);
            args.glist = (int32_t *)((char *)workspace + pad256(off));
            args.glist_cap = glist_cap(slots, d->num_seqs);
        }
    }
    if (d->num_seqs > 0) {
        void *outs[6] = {dr, dw, dk, dv, da, db};
        if (wkv7::launch_zero_uncovered(args.seg, d->grad_f32 ? WKV7_F32 : d->dtype, outs, 6, hs) != hipSuccess)
            return WKV7_ERR_HIP;
    }
    if (wkv7::launch_backward_sweep(args, hs) != hipSuccess) return WKV7_ERR_HIP;
    if (wkv7::launch_backward(args, hs) != hipSuccess) return WKV7_ERR_HIP;
    return WKV7_OK;
}

wkv7_status wkv7_backward(const wkv7_desc *d, const void *r, const void *w, const void *k,
                          const void *v, const void *a, const void *b, const float *ckpt,
                          const void *dy, const float *ds_out, void *dr, void *dw, void *dk,
                          void *dv, void *da, void *db, float *ds0, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return backward_impl(d, r, w, k, v, a, b, ckpt, dy, ds_out, dr, dw, dk, dv, da, db, ds0,
                         workspace, workspace_bytes, false, stream);
}

wkv7_status wkv7_backward_noalloc(const wkv7_desc *d, const void *r, const void *w, const void *k,
                                  const void *v, const void *a, const void *b, const float *ckpt,
                                  const void *dy, const float *ds_out, void *dr, void *dw, void *dk,
                                  void *dv, void *da, void *db, float *ds0, void *stream) {
    return backward_impl(d, r, w, k, v, a, b, ckpt, dy, ds_out, dr, dw, dk, dv, da, db, ds0,
                         nullptr, 0, true, stream);
}

static wkv7_status decode_impl(int32_t B, int32_t H, int32_t N, int32_t dtype, int32_t decay,
                               const void *r, const void *w, const void *k, const void *v,
                               const void *a, const void *b, const float *s_in, float *s_out,
                               void *y, const void *g, const float *ln_w, const float *ln_b,
                               const float *r_k, float eps, void *out, void *stream) {
    const bool fused = out != nullptr;
    if (N != kN && (fused || N != 128)) return WKV7_ERR_UNSUPPORTED;   // 128: plain step only
    if (!dtype_ok(dtype)) return WKV7_ERR_UNSUPPORTED;
    if (decay != WKV7_DECAY_MULT && decay != WKV7_DECAY_LOG) return WKV7_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || (int64_t)B * H > INT32_MAX) return WKV7_ERR_INVALID_ARGUMENT;
    const void *streams[9] = {r, w, k, v, a, b, fused ? out : y, s_in, s_out};
    wkv7_status st = check_streams(streams, 9);
    if (st != WKV7_OK) return st;
    if (fused) {
        const void *params[4] = {g, ln_w, ln_b, r_k};
        if ((st = check_streams(params, 4)) != WKV7_OK) return st;
        if (y && !aligned16(y)) return WKV7_ERR_INVALID_ARGUMENT;
        if (!(eps >= 0.f) || !std::isfinite(eps)) return WKV7_ERR_INVALID_ARGUMENT;
    }
    const size_t state_bytes = (size_t)B * H * N * N * sizeof(float);
    if (s_in != s_out && ranges_overlap(s_in, state_bytes, s_out, state_bytes))
        return WKV7_ERR_INVALID_ARGUMENT;
    {
        // in place (s_out == s_in) the state is an output only
        const size_t tb = (size_t)B * H * N * elem_size(dtype), pb = (size_t)H * N * sizeof(float);
        const Range ins[11] = {{r, tb}, {w, tb}, {k, tb}, {v, tb}, {a, tb}, {b, tb},
                               {s_in == s_out ? nullptr : s_in, state_bytes},
                               {fused ? g : nullptr, tb}, {fused ? ln_w : nullptr, pb},
                               {fused ? ln_b : nullptr, pb}, {fused ? r_k : nullptr, pb}};
        const Range outs[3] = {{s_out, state_bytes}, {y, tb}, {fused ? out : nullptr, tb}};
        if (any_overlap(ins, 11, outs, 3)) return WKV7_ERR_INVALID_ARGUMENT;
    }
    if ((st = check_device()) != WKV7_OK) return st;
    wkv7::DecArgs args{};
    args.B = B; args.H = H; args.dtype = dtype;
    args.logw = decay == WKV7_DECAY_LOG;
    args.r = r; args.w = w; args.k = k; args.v = v; args.a = a; args.b = b;
    args.s_in = s_in; args.s_out = s_out; args.y = y;
    if (fused) {
        args.g = g; args.ln_w = ln_w; args.ln_b = ln_b; args.r_k = r_k;
        args.eps = eps; args.out = out;
    }
    const hipError_t e = N == 128 ? wkv7::launch_decode128(args, (hipStream_t)stream)
                                  : wkv7::launch_decode(args, (hipStream_t)stream);
    if (e != hipSuccess) return WKV7_ERR_HIP;
    return WKV7_OK;
}

wkv7_status wkv7_decode_step(int32_t B, int32_t H, int32_t N, int32_t dtype, int32_t decay,
                             const void *r,
                             const void *w, const void *k, const void *v, const void *a,
                             const void *b, const float *s_in, float *s_out, void *y,
                             void *stream) {
    return decode_impl(B, H, N, dtype, decay, r, w, k, v, a, b, s_in, s_out, y,
                       nullptr, nullptr, nullptr, nullptr, 0.f, nullptr, stream);
}

wkv7_status wkv7_decode_step_fused(int32_t B, int32_t H, int32_t N, int32_t dtype, int32_t decay,
                                   const void *r, const void *w, const void *k, const void *v,
                                   const void *a, const void *b, const float *s_in, float *s_out,
                                   const void *g, const float *ln_w, const float *ln_b,
                                   const float *r_k, float eps, void *out, void *y, void *stream) {
    if (!out) return WKV7_ERR_INVALID_ARGUMENT;
    return decode_impl(B, H, N, dtype, decay, r, w, k, v, a, b, s_in, s_out, y,
                       g, ln_w, ln_b, r_k, eps, out, stream);
}

wkv7_status wkv7_gdn_decode_step(int32_t B, int32_t H, int32_t Hk, int32_t N, int32_t dtype,
                                 const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *s_in, float *s_out, void *out,
                                 void *stream) {
    if (N != 64 && N != 128) return WKV7_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return WKV7_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Hk < 1 || H % Hk != 0 || (int64_t)B * H > INT32_MAX)
        return WKV7_ERR_INVALID_ARGUMENT;
    const void *streams[6] = {q, k, v, s_in, s_out, out};
    wkv7_status st = check_streams(streams, 6);
    if (st != WKV7_OK) return st;
    if (!g || !beta || !aligned4(g) || !aligned4(beta)) return WKV7_ERR_INVALID_ARGUMENT;
    const size_t state_bytes = (size_t)B * H * N * N * sizeof(float);
    if (s_in != s_out && ranges_overlap(s_in, state_bytes, s_out, state_bytes))
        return WKV7_ERR_INVALID_ARGUMENT;
    {
        const size_t es = elem_size(dtype);
        const size_t qb = (size_t)B * Hk * N * es, vb = (size_t)B * H * N * es, sc = (size_t)B * H * 4;
        const Range ins[6] = {{q, qb}, {k, qb}, {v, vb}, {g, sc}, {beta, sc},
                              {s_in == s_out ? nullptr : s_in, state_bytes}};
        const Range outs[2] = {{s_out, state_bytes}, {out, vb}};
        if (any_overlap(ins, 6, outs, 2)) return WKV7_ERR_INVALID_ARGUMENT;
    }
    if ((st = check_device()) != WKV7_OK) return st;
    wkv7::GdnArgs a{};
    a.B = B; a.H = H; a.Hk = Hk; a.N = N; a.dtype = dtype;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s_in = s_in; a.s_out = s_out; a.out = out;
    if (wkv7::launch_gdn_decode(a, (hipStream_t)stream) != hipSuccess) return WKV7_ERR_HIP;
    return WKV7_OK;
}

wkv7_status wkv7_gdn_workspace_bytes(int32_t B, int32_t T, int32_t Hk, int32_t N, size_t *bytes) {
    if (N != 64 && N != 128) return WKV7_ERR_UNSUPPORTED;
    // the row pre-pass takes 4 token rows per 256-thread workgroup
    if (B < 1 || T < 1 || Hk < 1 || (int64_t)B * T * Hk > (1 << 24)) return WKV7_ERR_INVALID_ARGUMENT;
    if (!bytes) return WKV7_ERR_INVALID_ARGUMENT;
    *bytes = 2 * pad256((size_t)B * T * Hk * N * sizeof(float));
    return WKV7_OK;
}

wkv7_status wkv7_gdn_forward(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t N, int32_t dtype,
                             const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *s0, void *out, float *s_out,
                             void *workspace, size_t workspace_bytes, void *stream) {
    size_t need = 0;
    wkv7_status st = wkv7_gdn_workspace_bytes(B, T, Hk, N, &need);
    if (st != WKV7_OK) return st;
    if (!dtype_ok(dtype)) return WKV7_ERR_UNSUPPORTED;
    // one N-lane workgroup per (sequence, value head)
    if (H < 1 || H % Hk != 0 || (int64_t)B * H > (1 << 24) || (int64_t)B * T * H * N > kMaxElems)
        return WKV7_ERR_INVALID_ARGUMENT;
    const void *streams[4] = {q, k, v, out};
    if ((st = check_streams(streams, 4)) != WKV7_OK) return st;
    if (!g || !beta || !aligned4(g) || !aligned4(beta)) return WKV7_ERR_INVALID_ARGUMENT;
    if ((s0 && !aligned16(s0)) || (s_out && !aligned16(s_out))) return WKV7_ERR_INVALID_ARGUMENT;
    if (!workspace || !aligned16(workspace)) return WKV7_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return WKV7_ERR_WORKSPACE_TOO_SMALL;
    const size_t es = elem_size(dtype);
    const size_t state_bytes = (size_t)B * H * N * N * sizeof(float);
    const size_t out_bytes = (size_t)B * T * H * N * es;
    const void *ins[6] = {q, k, v, g, beta, s0};
    const size_t in_bytes[6] = {(size_t)B * T * Hk * N * es, (size_t)B * T * Hk * N * es, out_bytes,
                                (size_t)B * T * H * 4, (size_t)B * T * H * 4, s0 ? state_bytes : 0};
    const void *outs[3] = {out, s_out, workspace};
    const size_t outs_bytes[3] = {out_bytes, s_out ? state_bytes : 0, need};
    for (int o = 0; o < 3; ++o) {
        if (!outs[o] || !outs_bytes[o]) continue;
        for (int q2 = 0; q2 < 6; ++q2)
            if (ins[q2] && in_bytes[q2] && ranges_overlap(ins[q2], in_bytes[q2], outs[o], outs_bytes[o]))
                return WKV7_ERR_INVALID_ARGUMENT;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (outs[o2] && outs_bytes[o2] && ranges_overlap(outs[o], outs_bytes[o], outs[o2], outs_bytes[o2]))
                return WKV7_ERR_INVALID_ARGUMENT;
    }
    if ((st = check_device()) != WKV7_OK) return st;
    wkv7::GdnFwdArgs a{};
    a.B = B; a.T = T; a.H = H; a.Hk = Hk; a.N = N; a.dtype = dtype;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.s0 = s0; a.out = out; a.s_out = s_out;
    a.qn = (float *)workspace;
    a.kn = (float *)((char *)workspace + need / 2);
    if (wkv7::launch_gdn_forward(a, (hipStream_t)stream) != hipSuccess) return WKV7_ERR_HIP;
    return WKV7_OK;
}

// Workspace of wkv7_gdn_backward, in 256-byte aligned parts: q^, k^
// ([B][T][Hk][N] fp32 each), the remapped streams r, w, k_w, v, a, b and dy
// and the WKV-7 gradients dr (first the discarded forward y), dw, dk, dv,
// da, db ([B][T][H][N] fp32 each), the checkpoints, and the WKV-7
// backward's own workspace.
struct GdnBwdLayout {
    size_t key, val, ckpt, wkv, total;
};
static wkv7_status gdn_bwd_layout(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t N, GdnBwdLayout *l) {
    size_t dummy = 0;
    wkv7_status st = wkv7_gdn_workspace_bytes(B, T, Hk, N, &dummy);
    if (st != WKV7_OK) return st;
    if (H < 1 || H % Hk != 0 || (int64_t)B * H > (1 << 24) || (int64_t)B * T * H * N > kMaxElems ||
        (int64_t)B * T > INT32_MAX || H > 65536)
        return WKV7_ERR_INVALID_ARGUMENT;
    wkv7_desc d{};
    d.B = B; d.T = T; d.H = H; d.N = N; d.dtype = WKV7_F32; d.grad_f32 = 1;
    size_t wkv = 0;
    if ((st = wkv7_workspace_bytes(&d, &wkv)) != WKV7_OK) return st;
    int64_t slots = 0;
    if ((st = wkv7_checkpoint_slots(B, T, &slots)) != WKV7_OK) return st;
    l->key = pad256((size_t)B * T * Hk * N * sizeof(float));
    l->val = pad256((size_t)B * T * H * N * sizeof(float));
    l->ckpt = pad256((size_t)slots * H * N * N * sizeof(float));
    l->wkv = pad256(wkv);
    l->total = 2 * l->key + 13 * l->val + l->ckpt + l->wkv;
    return WKV7_OK;
}

wkv7_status wkv7_gdn_backward_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t N,
                                              size_t *bytes) {
    GdnBwdLayout l;
    const wkv7_status st = gdn_bwd_layout(B, T, H, Hk, N, &l);
    if (st != WKV7_OK) return st;
    if (!bytes) return WKV7_ERR_INVALID_ARGUMENT;
    *bytes = l.total;
    return WKV7_OK;
}

wkv7_status wkv7_gdn_backward(int32_t B, int32_t T, int32_t H, int32_t Hk, int32_t N, int32_t dtype,
                              const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *s0, const void *dout, const float *ds_out,
                              void *dq, void *dk, void *dv, float *dg, float *dbeta, float *ds0,
                              void *workspace, size_t workspace_bytes, void *stream) {
    GdnBwdLayout l;
    wkv7_status st = gdn_bwd_layout(B, T, H, Hk, N, &l);
    if (st != WKV7_OK) return st;
    if (!dtype_ok(dtype)) return WKV7_ERR_UNSUPPORTED;
    const void *streams[6] = {q, k, v, dq, dk, dv};
    if ((st = check_streams(streams, 6)) != WKV7_OK) return st;
    if (dout && !aligned16(dout)) return WKV7_ERR_INVALID_ARGUMENT;
    if (!g || !beta || !dg || !dbeta || !aligned4(g) || !aligned4(beta) || !aligned4(dg) || !aligned4(dbeta))
        return WKV7_ERR_INVALID_ARGUMENT;
    if ((s0 && !aligned16(s0)) || (ds_out && !aligned16(ds_out)) || (ds0 && !aligned16(ds0)))
        return WKV7_ERR_INVALID_ARGUMENT;
    if (!workspace || !aligned16(workspace)) return WKV7_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < l.total) return WKV7_ERR_WORKSPACE_TOO_SMALL;
    {
        const size_t es = elem_size(dtype);
        const size_t kb = (size_t)B * T * Hk * N * es, vb = (size_t)B * T * H * N * es;
        const size_t sb = (size_t)B * T * H * sizeof(float), state = (size_t)B * H * N * N * sizeof(float);
        const Range ins[8] = {{q, kb}, {k, kb}, {v, vb}, {g, sb}, {beta, sb}, {s0, state}, {dout, vb},
                              {ds_out, state}};
        const Range outs[7] = {{dq, kb}, {dk, kb}, {dv, vb}, {dg, sb}, {dbeta, sb}, {ds0, state},
                               {workspace, l.total}};
        if (any_overlap(ins, 8, outs, 7)) return WKV7_ERR_INVALID_ARGUMENT;
    }
    if ((st = check_device()) != WKV7_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    char *ws = (char *)workspace;
    auto part = [&](size_t &off, size_t n) { float *x = (float *)(ws + off); off += n; return x; };
    size_t off = 0;
    wkv7::GdnBwdArgs a{};
    a.B = B; a.T = T; a.H = H; a.Hk = Hk; a.N = N; a.dtype = dtype;
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.g = g; a.beta = beta;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta;
    a.qn = part(off, l.key); a.kn = part(off, l.key);
    a.r = part(off, l.val); a.w = part(off, l.val); a.kw = part(off, l.val); a.v32 = part(off, l.val);
    a.a = part(off, l.val); a.b = part(off, l.val); a.dy = part(off, l.val);
    float *gr = part(off, l.val), *gw = part(off, l.val), *gk = part(off, l.val);
    float *gv = part(off, l.val), *ga = part(off, l.val), *gb = part(off, l.val);
    a.gr = gr; a.gw = gw; a.gk = gk; a.gv = gv; a.ga = ga; a.gb = gb;
    float *ckpt = part(off, l.ckpt);
    void *wkv_ws = l.wkv ? (void *)(ws + off) : nullptr;
    if (wkv7::launch_gdn_remap(a, hs) != hipSuccess) return WKV7_ERR_HIP;
    wkv7_desc d{};
    d.B = B; d.T = T; d.H = H; d.N = N; d.dtype = WKV7_F32; d.grad_f32 = 1;
    if (dtype == WKV7_BF16) {
        // the checkpoints from the GDN chunk form on q^, k^ (remap's pre-pass)
        // and the bf16 v: the same states as the remapped WKV-7 forward's
        wkv7::GdnFwdArgs f{};
        f.B = B; f.T = T; f.H = H; f.Hk = Hk; f.N = N; f.dtype = dtype;
        f.v = v; f.g = g; f.beta = beta; f.s0 = s0; f.qn = a.qn; f.kn = a.kn; f.ckpt = ckpt;
        if (wkv7::launch_gdn_forward_cf(f, hs) != hipSuccess) return WKV7_ERR_HIP;
    } else {
        // the forward for the checkpoints; its y goes to dr's part, which the
        // backward overwrites
        if ((st = wkv7_forward(&d, a.r, a.w, a.kw, a.v32, a.a, a.b, s0, gr, nullptr, ckpt, stream)) != WKV7_OK)
            return st;
    }
    if ((st = wkv7_backward(&d, a.r, a.w, a.kw, a.v32, a.a, a.b, ckpt, dout ? a.dy : nullptr, ds_out, gr, gw,
                            gk, gv, ga, gb, ds0, wkv_ws, l.wkv, stream)) != WKV7_OK)
        return st;
    if (wkv7::launch_gdn_pullback(a, hs) != hipSuccess) return WKV7_ERR_HIP;
    return WKV7_OK;
}

wkv7_status vce_forward_workspace_bytes(int32_t M, int32_t D, int32_t V, size_t *bytes) {
    wkv7_status st = vce_check_sizes(M, D, V);
    if (st != WKV7_OK) return st;
    if (!bytes) return WKV7_ERR_INVALID_ARGUMENT;
    *bytes = vce_fwd_bytes(M, V);
    return WKV7_OK;
}

wkv7_status vce_backward_workspace_bytes(int32_t M, int32_t D, int32_t V, int32_t vocab_chunk,
                                         size_t *bytes) {
    VceBwdLayout l;
    wkv7_status st = vce_bwd_layout(M, D, V, vocab_chunk, &l);
    if (st != WKV7_OK) return st;
    if (!bytes) return WKV7_ERR_INVALID_ARGUMENT;
    *bytes = l.total;
    return WKV7_OK;
}

wkv7_status vce_forward(int32_t M, int32_t D, int32_t V, const void *h, const void *w,
                        const int32_t *targets, float *loss, float *lse, void *workspace,
                        size_t workspace_bytes, void *stream) {
    wkv7_status st = vce_check_sizes(M, D, V);
    if (st != WKV7_OK) return st;
    if (!h || !w || !aligned16(h) || !aligned16(w)) return WKV7_ERR_INVALID_ARGUMENT;
    if (!targets || !loss || !lse || !aligned4(targets) || !aligned4(loss) || !aligned4(lse))
        return WKV7_ERR_INVALID_ARGUMENT;
    if (!workspace || !aligned16(workspace)) return WKV7_ERR_INVALID_ARGUMENT;
    const size_t need = vce_fwd_bytes(M, V);
    if (workspace_bytes < need) return WKV7_ERR_WORKSPACE_TOO_SMALL;
    const size_t row = (size_t)M * 4;
    if (ranges_overlap(loss, row, lse, row)) return WKV7_ERR_INVALID_ARGUMENT;
    const void *ins[3] = {h, w, targets};
    const size_t in_bytes[3] = {(size_t)M * D * 2, (size_t)V * D * 2, row};
    for (int q = 0; q < 3; ++q)
        if (ranges_overlap(ins[q], in_bytes[q], loss, row) || ranges_overlap(ins[q], in_bytes[q], lse, row) ||
            ranges_overlap(ins[q], in_bytes[q], workspace, need))
            return WKV7_ERR_INVALID_ARGUMENT;
    if (ranges_overlap(loss, row, workspace, need) || ranges_overlap(lse, row, workspace, need))
        return WKV7_ERR_INVALID_ARGUMENT;
    if ((st = check_device()) != WKV7_OK) return st;
    const vce::FwdPlan f = vce::fwd_plan(M, V);
    vce::FwdArgs a;
    a.M = M; a.D = D; a.V = V;
    a.h = (const uint16_t *)h; a.w = (const uint16_t *)w;
    a.targets = targets; a.loss = loss; a.lse = lse;
    a.part = (float2 *)workspace;
    a.zt = (float *)((char *)workspace + pad256((size_t)f.nsplit * M * 8));
    if (vce::launch_forward(a, (hipStream_t)stream) != hipSuccess) return WKV7_ERR_HIP;
    return WKV7_OK;
}

wkv7_status vce_backward(int32_t M, int32_t D, int32_t V, int32_t vocab_chunk, const void *h,
                         const void *w, const int32_t *targets, const float *lse,
                         const float *dloss, float *dh, float *dw, void *workspace,
                         size_t workspace_bytes, void *stream) {
    VceBwdLayout l;
    wkv7_status st = vce_bwd_layout(M, D, V, vocab_chunk, &l);
    if (st != WKV7_OK) return st;
    if (!h || !w || !aligned16(h) || !aligned16(w)) return WKV7_ERR_INVALID_ARGUMENT;
    if (!targets || !lse || !dloss || !dh || !dw) return WKV7_ERR_INVALID_ARGUMENT;
    if (!aligned4(targets) || !aligned4(lse) || !aligned4(dloss) || !aligned4(dh) || !aligned4(dw))
        return WKV7_ERR_INVALID_ARGUMENT;
    if (!workspace || !aligned16(workspace)) return WKV7_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < l.total) return WKV7_ERR_WORKSPACE_TOO_SMALL;
    const size_t row = (size_t)M * 4;
    const void *ins[5] = {h, w, targets, lse, dloss};
    const size_t in_bytes[5] = {(size_t)M * D * 2, (size_t)V * D * 2, row, row, row};
    void *outs[3] = {dh, dw, workspace};
    const size_t out_bytes[3] = {(size_t)M * D * 4, (size_t)V * D * 4, l.total};
    for (int o = 0; o < 3; ++o) {
        for (int q = 0; q < 5; ++q)
            if (ranges_overlap(ins[q], in_bytes[q], outs[o], out_bytes[o])) return WKV7_ERR_INVALID_ARGUMENT;
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (ranges_overlap(outs[o], out_bytes[o], outs[o2], out_bytes[o2])) return WKV7_ERR_INVALID_ARGUMENT;
    }
    if ((st = check_device()) != WKV7_OK) return st;
    char *ws = (char *)workspace;
    vce::BwdArgs a;
    a.M = M; a.D = D; a.V = V; a.Vc = l.Vc;
    a.h = (const uint16_t *)h; a.w = (const uint16_t *)w;
    a.targets = targets; a.lse = lse; a.dloss = dloss; a.dh = dh; a.dw = dw;
    a.wt = (uint16_t *)(ws + l.wt); a.ht = (uint16_t *)(ws + l.ht);
    a.g = (uint16_t *)(ws + l.g); a.gt = (uint16_t *)(ws + l.gt);
    if (vce::launch_backward(a, (hipStream_t)stream) != hipSuccess) return WKV7_ERR_HIP;
    return WKV7_OK;
}

}  // extern "C"
