// api.cpp -- the C ABI declared in include/flamia.h: host-side validation,
// workspace layout and kernel launches.  No device memory is allocated and no
// device memory is read on the host; every call only enqueues kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "flamia.h"
#include "kernels.hpp"

namespace {

using namespace flamia;

constexpr size_t kAlign = 256;
constexpr int kFwdTile = 128;  // queries per forward work item
constexpr int kBwdTile = 128;  // keys per backward work item (exact-scale modes)
constexpr int kBwdWideTile = 256;  // keys per backward work item (token-block operands)
// The 256-key backward splits its costliest items in two (see the work-list
// kernel); each split (item, kv head) pair keeps two FP32 slots of its raw
// dK / dV (256 keys x d x 2 tensors).  The slots take at most this many bytes.
constexpr size_t kSplitSlotBytes = (size_t)64 << 20;
constexpr int64_t kSplitMinIters = 64;
constexpr uint32_t kKnownFlags =
    FLAMIA_CAUSAL | FLAMIA_EXACT | FLAMIA_FP4_SCORE | FLAMIA_DETERMINISTIC | FLAMIA_HADAMARD |
    FLAMIA_DQ_PRESCALE_SEQUENCE;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Dims {
    int64_t T, B, Hq, Hkv, d;
    float scale;
    bool causal, deterministic, rotate;
};

flamia_status check_seq(const flamia_problem* p)
{
    if (p == nullptr) return FLAMIA_ERR_INVALID_ARG;
    if (p->total_tokens < 0 || p->num_seqs < 1 || p->cu_seqlens == nullptr)
        return FLAMIA_ERR_INVALID_ARG;
    return FLAMIA_OK;
}

flamia_status check_head_dim(int32_t d)
{
    if (d <= 0) return FLAMIA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FLAMIA_ERR_UNSUPPORTED;
    return FLAMIA_OK;
}

// The E2M1 score-view pointers are required with FLAMIA_FP4_SCORE and must
// be NULL without it.
flamia_status check_fp4_pointers(const flamia_problem* p, const void* q4, const void* q4s,
                                 const void* k4, const void* k4s)
{
    if (p->flags & FLAMIA_FP4_SCORE)
        return (q4 && q4s && k4 && k4s) ? FLAMIA_OK : FLAMIA_ERR_INVALID_ARG;
    return (q4 || q4s || k4 || k4s) ? FLAMIA_ERR_INVALID_ARG : FLAMIA_OK;
}

int operand_mode(const flamia_problem* p)
{
    if (p->flags & FLAMIA_FP4_SCORE) return MODE_FP4;
    return (p->flags & FLAMIA_EXACT) ? MODE_EXACT : MODE_BLOCK;
}

flamia_status check_attn(const flamia_problem* p, Dims* out)
{
    flamia_status st = check_seq(p);
    if (st != FLAMIA_OK) return st;
    if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_q_heads % p->num_kv_heads != 0)
        return FLAMIA_ERR_INVALID_ARG;
    // the dO preparation launches a 1-D grid of (32-token window, head)
    // workgroups of 256 threads
    if ((int64_t)(p->total_tokens + 31) / 32 * p->num_q_heads >= ((int64_t)1 << 24))
        return FLAMIA_ERR_UNSUPPORTED;
    st = check_head_dim(p->head_dim);
    if (st != FLAMIA_OK) return st;
    if (p->flags & ~kKnownFlags) return FLAMIA_ERR_INVALID_ARG;
    if ((p->flags & FLAMIA_FP4_SCORE) && !(p->flags & FLAMIA_EXACT)) return FLAMIA_ERR_INVALID_ARG;
    if ((p->flags & FLAMIA_HADAMARD) && (p->flags & FLAMIA_EXACT)) return FLAMIA_ERR_UNSUPPORTED;
    if (std::isnan(p->softmax_scale) || std::isinf(p->softmax_scale)) return FLAMIA_ERR_INVALID_ARG;
    out->T = p->total_tokens;
    out->B = p->num_seqs;
    out->Hq = p->num_q_heads;
    out->Hkv = p->num_kv_heads;
    out->d = p->head_dim;
    out->scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
    // rotated Q and K: q_r . k_r = d q . k (unnormalised Sylvester matrix), so
    // every use of the scale takes scale / d (exact: d is a power of two)
    if (p->flags & FLAMIA_HADAMARD) out->scale /= (float)p->head_dim;
    out->rotate = (p->flags & FLAMIA_HADAMARD) != 0;
    out->causal = (p->flags & FLAMIA_CAUSAL) != 0;
    out->deterministic = (p->flags & FLAMIA_DETERMINISTIC) != 0;
    // grid limits: items x heads must fit a 1-D launch
    const int64_t items = out->T / 128 + std::min(out->B, out->T) + 1;
    if (items * out->Hq >= (int64_t)INT32_MAX) return FLAMIA_ERR_UNSUPPORTED;
    return FLAMIA_OK;
}

int64_t max_items(const Dims& d, int tile) { return d.T / tile + std::min(d.B, d.T) + 1; }
int64_t max_cost(const Dims& d) { return (d.T + 63) / 64 + 1; }

struct WorklistLayout {
    size_t doc_off, hist, cursor, count, items, total;
};

WorklistLayout worklist_layout(const Dims& d, int tile, size_t base)
{
    WorklistLayout w;
    size_t o = base;
    w.doc_off = o;
    o = align_up(o + 4 * (size_t)(d.B + 1));
    w.hist = o;
    o = align_up(o + 4 * (size_t)(max_cost(d) + 1));
    w.cursor = o;
    o = align_up(o + 4 * (size_t)(max_cost(d) + 1));
    w.count = o;
    o = align_up(o + 4 * 3);
    w.items = o;
    o = align_up(o + 8 * (size_t)max_items(d, tile));
    w.total = o;
    return w;
}

// Split pairs of the 256-key backward (item x kv head) that the slots can
// hold, and the bytes of one pair's two slots.
size_t split_pair_bytes(const Dims& d) { return 2 * 2 * (size_t)kBwdWideTile * d.d * 4; }
int64_t split_pairs(const Dims& d)
{
    return std::min<int64_t>(max_items(d, kBwdWideTile) * d.Hkv,
                             (int64_t)(kSplitSlotBytes / split_pair_bytes(d)));
}

// The public part of the backward workspace layout, plus where its work lists
// (and, after them, the split pairs' counters and slots) start.
flamia_bwd_workspace_layout bwd_layout(const Dims& d, size_t* worklist_base = nullptr)
{
    flamia_bwd_workspace_layout l;
    const size_t rows = (size_t)d.T * d.Hq;
    size_t o = 0;
    l.do_codes = o;
    o = align_up(o + rows * d.d);
    l.do_exps = o;
    o = align_up(o + rows);
    l.delta = o;
    o = align_up(o + 4 * rows);
    l.dq_prescale = o;
    o = align_up(o + rows);
    l.dq_accum = o;
    o = align_up(o + 2 * rows * d.d);
    if (worklist_base) *worklist_base = o;
    o = worklist_layout(d, kBwdTile, o).total;
    if (worklist_base) worklist_base[1] = o;  // query-tile list of the deterministic dQ kernel
    o = worklist_layout(d, kFwdTile, o).total;
    if (worklist_base) worklist_base[2] = o;  // the split pairs' slots
    l.total = o + split_pairs(d) * split_pair_bytes(d);
    return l;
}

WorklistArgs make_worklist_args(const Dims& d, const flamia_problem* p, int tile, bool backward,
                                uint8_t* ws, const WorklistLayout& w)
{
    WorklistArgs a = {};
    a.B = (int)d.B;
    a.T = (int)d.T;
    a.tile = tile;
    a.causal = d.causal ? 1 : 0;
    a.backward = backward ? 1 : 0;
    a.max_items = (int)max_items(d, tile);
    a.max_cost = (int)max_cost(d);
    a.cu = p->cu_seqlens;
    a.doc_off = (int32_t*)(ws + w.doc_off);
    a.hist = (int32_t*)(ws + w.hist);
    a.cursor = (int32_t*)(ws + w.cursor);
    a.count = (int32_t*)(ws + w.count);
    a.items = (int32_t*)(ws + w.items);
    return a;
}

// C of the dQ prescale: ceil(log2(4 * scale * d * 448^3)).
int prescale_c(const Dims& d)
{
    return (int)std::ceil(std::log2(4.0 * (double)d.scale * (double)d.d * 448.0 * 448.0 * 448.0));
}

flamia_status hip_status(hipError_t e) { return e == hipSuccess ? FLAMIA_OK : FLAMIA_ERR_HIP; }

// The caller's timing events, if any, for the launch of the call's main
// kernel (recorded around its launch, see AttnArgs).
void set_events(const flamia_problem* p, hipEvent_t& start, hipEvent_t& stop)
{
    start = p->events ? (hipEvent_t)p->events->attn_start : nullptr;
    stop = p->events ? (hipEvent_t)p->events->attn_stop : nullptr;
}

constexpr size_t kNoallocScratchBytes = size_t(4) << 20;

}  // namespace

// Scratch of the allocation-free forward (flamia_attn_fwd_noalloc): its work
// list lives in this fixed device array instead of a caller's workspace.
// Every GPU the library runs on holds its own copy until the process ends,
// and every call on a GPU shares it (calls that overlap on one GPU race).
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

// The device address of `scratch` on each device, looked up once per device
// with that device current.  (The name `scratch` in host code is a host-side
// stand-in, not a device address.)
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

flamia_status scratch_of_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FLAMIA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FLAMIA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return FLAMIA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FLAMIA_OK;
}

flamia_status attn_fwd_impl(const flamia_problem* p, const uint8_t* q_codes,
                              const uint8_t* q_exps, const uint8_t* k_codes,
                              const uint8_t* k_exps, const uint8_t* v_codes,
                              const uint8_t* v_exps, const uint8_t* q_fp4,
                              const uint8_t* q_fp4_scales, const uint8_t* k_fp4,
                              const uint8_t* k_fp4_scales, uint16_t* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream)
{
    Dims d;
    flamia_status st = check_attn(p, &d);
    if (st != FLAMIA_OK) return st;
    st = check_fp4_pointers(p, q_fp4, q_fp4_scales, k_fp4, k_fp4_scales);
    if (st != FLAMIA_OK) return st;
    if (d.T == 0) return FLAMIA_OK;
    if (!q_codes || !q_exps || !k_codes || !k_exps || !v_codes || !v_exps || !o || !lse)
        return FLAMIA_ERR_INVALID_ARG;
    const WorklistLayout wl = worklist_layout(d, kFwdTile, 0);
    if (workspace == nullptr || workspace_bytes < wl.total) return FLAMIA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;

    WorklistArgs w = make_worklist_args(d, p, kFwdTile, false, ws, wl);
    hipError_t e = launch_worklist(w, s);
    if (e != hipSuccess) return FLAMIA_ERR_HIP;

    AttnArgs a = {};
    a.T = (int)d.T;
    a.B = (int)d.B;
    a.Hq = (int)d.Hq;
    a.Hkv = (int)d.Hkv;
    a.causal = d.causal ? 1 : 0;
    a.scale = d.scale;
    a.c2 = d.scale * 1.4426950408889634f;
    a.cu = p->cu_seqlens;
    a.count = w.count;
    a.items = w.items;
    a.q_codes = q_codes;
    a.q_exps = q_exps;
    a.k_codes = k_codes;
    a.k_exps = k_exps;
    a.v_codes = v_codes;
    a.v_exps = v_exps;
    a.mode = operand_mode(p);
    a.rotate = d.rotate ? 1 : 0;
    a.q_fp4 = q_fp4;
    a.q_fp4_scales = q_fp4_scales;
    a.k_fp4 = k_fp4;
    a.k_fp4_scales = k_fp4_scales;
    a.o = o;
    a.lse = lse;
    set_events(p, a.ev_start, a.ev_stop);
    return hip_status(launch_fwd(a, (int)d.d, w.max_items, s));
}

}  // namespace

extern "C" {

const char* flamia_status_string(flamia_status s)
{
    switch (s) {
    case FLAMIA_OK: return "ok";
    case FLAMIA_ERR_INVALID_ARG: return "invalid argument";
    case FLAMIA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FLAMIA_ERR_WORKSPACE: return "workspace missing or too small";
    case FLAMIA_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

flamia_status flamia_quantize_tokblock(const flamia_problem* p, int32_t num_heads,
                                       int32_t scale_mode, const uint16_t* x, uint8_t* codes,
                                       uint8_t* exps, void* stream)
{
    flamia_status st = check_seq(p);
    if (st != FLAMIA_OK) return st;
    st = check_head_dim(p->head_dim);
    if (st != FLAMIA_OK) return st;
    if (num_heads < 1) return FLAMIA_ERR_INVALID_ARG;
    const bool rotate = (scale_mode & FLAMIA_SCALE_ROTATE) != 0;
    const bool floor_rule = (scale_mode & FLAMIA_SCALE_FLOOR_CONTROL) != 0;
    scale_mode &= ~(int32_t)(FLAMIA_SCALE_ROTATE | FLAMIA_SCALE_FLOOR_CONTROL);
    if (scale_mode != FLAMIA_SCALE_TOKBLOCK32 && scale_mode != FLAMIA_SCALE_PER_TOKEN &&
        scale_mode != FLAMIA_SCALE_NVFP4_16)
        return FLAMIA_ERR_INVALID_ARG;
    if ((rotate || floor_rule) && scale_mode == FLAMIA_SCALE_NVFP4_16) return FLAMIA_ERR_INVALID_ARG;
    // 1-D grid of (32-token window, head) workgroups of 256 threads; the
    // E2M1 view launches one thread per 16 features
    if ((int64_t)(p->total_tokens + 31) / 32 * num_heads >= ((int64_t)1 << 24))
        return FLAMIA_ERR_UNSUPPORTED;
    if ((int64_t)p->total_tokens * num_heads * (p->head_dim / 16) >= ((int64_t)1 << 32) - 256)
        return FLAMIA_ERR_UNSUPPORTED;
    if (p->total_tokens == 0) return FLAMIA_OK;
    if (x == nullptr || codes == nullptr || exps == nullptr) return FLAMIA_ERR_INVALID_ARG;
    QuantArgs a = {};
    a.T = p->total_tokens;
    a.B = p->num_seqs;
    a.H = num_heads;
    a.block = scale_mode == FLAMIA_SCALE_PER_TOKEN ? 1 : 32;
    a.rotate = rotate ? 1 : 0;
    a.floor_rule = floor_rule ? 1 : 0;
    a.ntensors = 1;
    a.Htot = num_heads;
    a.ten[0] = QuantTensor{x, codes, exps, num_heads, rotate ? 1 : 0};
    a.cu = p->cu_seqlens;
    a.x = x;
    a.codes = codes;
    a.exps = exps;
    hipStream_t s = (hipStream_t)stream;
    set_events(p, a.ev_start, a.ev_stop);
    const hipError_t e = scale_mode == FLAMIA_SCALE_NVFP4_16 ? launch_nvfp4(a, p->head_dim, s)
                                                             : launch_quant(a, p->head_dim, false, s);
    return hip_status(e);
}

flamia_status flamia_quantize_qkv(const flamia_problem* p, int32_t scale_mode, const uint16_t* q,
                                  const uint16_t* k, const uint16_t* v, uint8_t* q_codes,
                                  uint8_t* q_exps, uint8_t* k_codes, uint8_t* k_exps,
                                  uint8_t* v_codes, uint8_t* v_exps, void* stream)
{
    flamia_status st = check_seq(p);
    if (st != FLAMIA_OK) return st;
    st = check_head_dim(p->head_dim);
    if (st != FLAMIA_OK) return st;
    const int Hq = p->num_q_heads, Hkv = p->num_kv_heads;
    if (Hq < 1 || Hkv < 1) return FLAMIA_ERR_INVALID_ARG;
    const bool rotate = (scale_mode & FLAMIA_SCALE_ROTATE) != 0;
    const bool floor_rule = (scale_mode & FLAMIA_SCALE_FLOOR_CONTROL) != 0;
    scale_mode &= ~(int32_t)(FLAMIA_SCALE_ROTATE | FLAMIA_SCALE_FLOOR_CONTROL);
    if (scale_mode != FLAMIA_SCALE_TOKBLOCK32 && scale_mode != FLAMIA_SCALE_PER_TOKEN)
        return FLAMIA_ERR_INVALID_ARG;
    const int64_t Htot = (int64_t)Hq + 2 * (int64_t)Hkv;
    if ((int64_t)(p->total_tokens + 31) / 32 * Htot >= ((int64_t)1 << 24)) return FLAMIA_ERR_UNSUPPORTED;
    if (p->total_tokens == 0) return FLAMIA_OK;
    if (!q || !k || !v || !q_codes || !q_exps || !k_codes || !k_exps || !v_codes || !v_exps)
        return FLAMIA_ERR_INVALID_ARG;
    QuantArgs a = {};
    a.T = p->total_tokens;
    a.B = p->num_seqs;
    a.block = scale_mode == FLAMIA_SCALE_PER_TOKEN ? 1 : 32;
    a.floor_rule = floor_rule ? 1 : 0;
    a.cu = p->cu_seqlens;
    a.ntensors = 3;
    a.Htot = (int)Htot;
    a.ten[0] = QuantTensor{q, q_codes, q_exps, Hq, rotate ? 1 : 0};
    a.ten[1] = QuantTensor{k, k_codes, k_exps, Hkv, rotate ? 1 : 0};
    a.ten[2] = QuantTensor{v, v_codes, v_exps, Hkv, 0};
    hipStream_t s = (hipStream_t)stream;
    set_events(p, a.ev_start, a.ev_stop);
    return hip_status(launch_quant(a, p->head_dim, false, s));
}

size_t flamia_attn_fwd_workspace_size(const flamia_problem* p)
{
    Dims d;
    if (check_attn(p, &d) != FLAMIA_OK) return 0;
    return worklist_layout(d, kFwdTile, 0).total;
}

flamia_status flamia_attn_fwd(const flamia_problem* p, const uint8_t* q_codes,
                              const uint8_t* q_exps, const uint8_t* k_codes,
                              const uint8_t* k_exps, const uint8_t* v_codes,
                              const uint8_t* v_exps, const uint8_t* q_fp4,
                              const uint8_t* q_fp4_scales, const uint8_t* k_fp4,
                              const uint8_t* k_fp4_scales, uint16_t* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream)
{
    return attn_fwd_impl(p, q_codes, q_exps, k_codes, k_exps, v_codes, v_exps, q_fp4, q_fp4_scales,
                         k_fp4, k_fp4_scales, o, lse, workspace, workspace_bytes, stream);
}

size_t flamia_attn_fwd_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

flamia_status flamia_attn_fwd_noalloc(const flamia_problem* p, const uint8_t* q_codes,
                                      const uint8_t* q_exps, const uint8_t* k_codes,
                                      const uint8_t* k_exps, const uint8_t* v_codes,
                                      const uint8_t* v_exps, const uint8_t* q_fp4,
                                      const uint8_t* q_fp4_scales, const uint8_t* k_fp4,
                                      const uint8_t* k_fp4_scales, uint16_t* o, float* lse,
                                      void* stream)
{
    Dims d;
    flamia_status st = check_attn(p, &d);
    if (st != FLAMIA_OK) return st;
    // the work list must fit the fixed scratch: rejected before any launch
    if (d.T > 0 && worklist_layout(d, kFwdTile, 0).total > kNoallocScratchBytes)
        return FLAMIA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (d.T > 0) {
        st = scratch_of_current_device(&ws);
        if (st != FLAMIA_OK) return st;
    }
    return attn_fwd_impl(p, q_codes, q_exps, k_codes, k_exps, v_codes, v_exps, q_fp4, q_fp4_scales,
                         k_fp4, k_fp4_scales, o, lse, ws, kNoallocScratchBytes, stream);
}

size_t flamia_attn_bwd_workspace_size(const flamia_problem* p)
{
    Dims d;
    if (check_attn(p, &d) != FLAMIA_OK) return 0;
    return bwd_layout(d).total;
}

flamia_status flamia_attn_bwd_workspace_layout(const flamia_problem* p,
                                               flamia_bwd_workspace_layout* out)
{
    Dims d;
    flamia_status st = check_attn(p, &d);
    if (st != FLAMIA_OK) return st;
    if (out == nullptr) return FLAMIA_ERR_INVALID_ARG;
    *out = bwd_layout(d);
    return FLAMIA_OK;
}

flamia_status flamia_attn_bwd(const flamia_problem* p, const uint8_t* q_codes,
                              const uint8_t* q_exps, const uint8_t* k_codes,
                              const uint8_t* k_exps, const uint8_t* v_codes,
                              const uint8_t* v_exps, const uint8_t* q_fp4,
                              const uint8_t* q_fp4_scales, const uint8_t* k_fp4,
                              const uint8_t* k_fp4_scales, const uint16_t* o, const float* lse,
                              const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                              void* workspace, size_t workspace_bytes, void* stream)
{
    Dims d;
    flamia_status st = check_attn(p, &d);
    if (st != FLAMIA_OK) return st;
    st = check_fp4_pointers(p, q_fp4, q_fp4_scales, k_fp4, k_fp4_scales);
    if (st != FLAMIA_OK) return st;
    // the deterministic dQ pass uses block exponents only and accumulates in
    // FP32 (no prescale); the FP16 view of the Q tile does not fit the
    // workgroup's LDS next to d = 128 tiles
    if ((p->flags & (FLAMIA_EXACT | FLAMIA_HADAMARD | FLAMIA_DQ_PRESCALE_SEQUENCE)) && d.deterministic)
        return FLAMIA_ERR_UNSUPPORTED;
    if ((p->flags & FLAMIA_FP4_SCORE) && d.d == 128) return FLAMIA_ERR_UNSUPPORTED;
    if (d.T == 0) return FLAMIA_OK;
    if (!q_codes || !q_exps || !k_codes || !k_exps || !v_codes || !v_exps || !o || !lse ||
        !dout || !dq || !dk || !dv)
        return FLAMIA_ERR_INVALID_ARG;
    size_t wl_base[3] = {0, 0, 0};
    const flamia_bwd_workspace_layout L = bwd_layout(d, wl_base);
    if (workspace == nullptr || workspace_bytes < L.total) return FLAMIA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;

    // dO quantization, D, prescale exponents, accumulator zeroing
    QuantArgs q = {};
    q.T = (int)d.T;
    q.B = (int)d.B;
    q.H = (int)d.Hq;
    q.block = (p->flags & FLAMIA_EXACT) ? 1 : 32;
    q.cu = p->cu_seqlens;
    q.x = dout;
    q.codes = ws + L.do_codes;
    q.exps = ws + L.do_exps;
    q.ntensors = 1;
    q.Htot = q.H;
    q.ten[0] = QuantTensor{dout, q.codes, q.exps, q.H, 0};
    q.Hkv = (int)d.Hkv;
    q.causal = d.causal ? 1 : 0;
    q.prescale_c = prescale_c(d);
    q.o = o;
    q.k_exps = k_exps;
    q.v_exps = v_exps;
    q.delta = (float*)(ws + L.delta);
    q.prescale = (int8_t*)(ws + L.dq_prescale);
    q.dq_acc = (_Float16*)(ws + L.dq_accum);
    hipError_t e = launch_quant(q, (int)d.d, true, s);
    if (e != hipSuccess) return FLAMIA_ERR_HIP;
    if (p->flags & FLAMIA_DQ_PRESCALE_SEQUENCE) {
        e = launch_seq_prescale(q, s);
        if (e != hipSuccess) return FLAMIA_ERR_HIP;
    }

    // 256-key tiles for token-block operands and for per-token operands at
    // d = 64; per-token operands at d = 128 keep 128-key tiles (the layout is
    // sized for the larger item count of 128-key tiles)
    const bool wide = operand_mode(p) == MODE_BLOCK || d.d == 64;
    const WorklistLayout wl = worklist_layout(d, kBwdTile, wl_base[0]);
    WorklistArgs w = make_worklist_args(d, p, wide ? kBwdWideTile : kBwdTile, true, ws, wl);
    if (wide) {
        w.split_wgs = bwd_wide_workgroups(2 * (int64_t)w.max_items * d.Hkv);
        if (w.split_wgs <= 0) return FLAMIA_ERR_HIP;
        w.split_cap = (int)(split_pairs(d) / d.Hkv);
        w.split_hkv = (int)d.Hkv;
        // a ticket of an item of cost c takes (Hq / Hkv) c iterations; split
        // only tickets of at least kSplitMinIters
        const int64_t G = d.Hq / d.Hkv;
        w.split_min_cost = (int)((kSplitMinIters + G - 1) / G);
    }
    e = launch_worklist(w, s);
    if (e != hipSuccess) return FLAMIA_ERR_HIP;

    AttnArgs a = {};
    a.T = (int)d.T;
    a.B = (int)d.B;
    a.Hq = (int)d.Hq;
    a.Hkv = (int)d.Hkv;
    a.causal = d.causal ? 1 : 0;
    a.scale = d.scale;
    a.c2 = d.scale * 1.4426950408889634f;
    {
        int ex = 0;
        const float m = std::frexp(d.scale, &ex);  // scale = m 2^ex, m in [0.5, 1)
        a.scale_exp = ex - 1;
        a.scale_res = 2.0f * m;
    }
    a.cu = p->cu_seqlens;
    a.count = w.count;
    a.tickets = w.count + 1;
    a.items = w.items;
    a.q_codes = q_codes;
    a.q_exps = q_exps;
    a.k_codes = k_codes;
    a.k_exps = k_exps;
    a.v_codes = v_codes;
    a.v_exps = v_exps;
    a.lse_in = lse;
    a.do_codes = q.codes;
    a.do_exps = q.exps;
    a.delta = q.delta;
    a.prescale = q.prescale;
    a.dq_acc = q.dq_acc;
    a.dkv_part = (float*)(ws + wl_base[2]);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.mode = operand_mode(p);
    a.rotate = d.rotate ? 1 : 0;
    a.q_fp4 = q_fp4;
    a.q_fp4_scales = q_fp4_scales;
    a.k_fp4 = k_fp4;
    a.k_fp4_scales = k_fp4_scales;
    set_events(p, a.ev_start, a.ev_stop);
    e = wide ? launch_bwd_wide(a, (int)d.d, w.max_items, !d.deterministic, s)
             : launch_bwd(a, (int)d.d, w.max_items, !d.deterministic, s);
    if (e != hipSuccess) return FLAMIA_ERR_HIP;
    a.ev_start = a.ev_stop = nullptr;
    if (d.deterministic) {
        // dQ by query-major blocks in FP32 registers, written directly
        const WorklistLayout wq = worklist_layout(d, kFwdTile, wl_base[1]);
        WorklistArgs wqa = make_worklist_args(d, p, kFwdTile, false, ws, wq);
        if (launch_worklist(wqa, s) != hipSuccess) return FLAMIA_ERR_HIP;
        AttnArgs aq = a;
        aq.count = wqa.count;
        aq.items = wqa.items;
        if (launch_bwd_dq(aq, (int)d.d, wqa.max_items, s) != hipSuccess) return FLAMIA_ERR_HIP;
    }
    if (wide && launch_bwd_pairs(a, (int)d.d, (int)split_pairs(d), s) != hipSuccess) return FLAMIA_ERR_HIP;
    return hip_status(launch_bwd_finalize(a, (int)d.d, !d.deterministic, s));
}

}  // extern "C"
