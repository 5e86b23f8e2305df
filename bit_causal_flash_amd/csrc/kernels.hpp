// kernels.hpp -- argument blocks and launchers of the HIP kernels (internal;
// the public interface is include/flamia.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flamia {

// A plain launch, bracketed by the caller's timing events when it asked for
// them (recorded on the same stream just before and after the launch).  The
// launch itself is the same either way: stamping the dispatch instead
// (hipExtLaunchKernel with events) was measured to slow the kernel down, by
// up to half of its time for the short d = 64 backward.
#define FLAMIA_LAUNCH(KERNEL, GRID, BLOCK, STREAM, EV0, EV1, ...)             \
    do {                                                                      \
        if ((EV0) != nullptr) (void)hipEventRecord(EV0, STREAM);              \
        hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, __VA_ARGS__);      \
        if ((EV1) != nullptr) (void)hipEventRecord(EV1, STREAM);              \
    } while (0)

// One tensor of a quantizer launch.
struct QuantTensor {
    const uint16_t* x;   // bf16 [T][H][D]
    uint8_t* codes;      // [T][H][D]
    uint8_t* exps;       // [H][T]
    int H;
    int rotate;          // Hadamard-rotate every row first (score operands)
};

struct QuantArgs {
    int T, B, H, block;
    // the token-block kernel: up to three tensors (Q, K, V) in one launch,
    // heads of all of them fastest; ten[0] alone for one tensor or dO
    int ntensors, Htot;
    QuantTensor ten[3];
    int rotate;          // Hadamard-rotate every row before quantizing (score operands)
    int floor_rule;      // floor exponent rule (negative control for the causality tests)
    const int32_t* cu;
    const uint16_t* x;   // bf16 [T][H][D]
    uint8_t* codes;      // [T][H][D]
    uint8_t* exps;       // [H][T]
    // backward preparation only
    int Hkv, causal, prescale_c;
    const uint16_t* o;        // bf16 [T][H][D]
    const uint8_t* k_exps;    // [Hkv][T]
    const uint8_t* v_exps;    // [Hkv][T]
    float* delta;             // [H][T]
    int8_t* prescale;         // [H][T]
    _Float16* dq_acc;         // [T][H][D]
    // optional: recorded just before / after the launch of the kernel
    hipEvent_t ev_start, ev_stop;
};

hipError_t launch_quant(const QuantArgs& a, int D, bool prep, hipStream_t stream);
// Sequence-wide dQ prescale (negative control): overwrites a.prescale after
// the backward preparation, from a.exps (dO), a.k_exps and a.v_exps
hipError_t launch_seq_prescale(const QuantArgs& a, hipStream_t stream);
// E2M1 + E4M3-per-16 score view: codes [T][H][D/2], scales (in exps) [T][H][D/16]
hipError_t launch_nvfp4(const QuantArgs& a, int D, hipStream_t stream);

// Work list of (document, tile) items sorted by decreasing cost.
struct WorklistArgs {
    int B, T, tile, causal, backward;
    int max_items, max_cost;
    const int32_t* cu;
    int32_t* doc_off;    // [B + 1]
    int32_t* hist;       // [max_cost + 1]
    int32_t* cursor;     // [max_cost + 1]
    int32_t* count;      // [3]: items, the persistent grid's ticket counter, items split in two
    int32_t* items;      // [max_items][2] = (doc, tile)
    // Backward 256-key list: the costliest items (a prefix of the order) are
    // split into two tickets per kv head when one ticket would take more
    // than half of a workgroup's average share.  split_cap: most items that
    // may be split (0: none); split_wgs: workgroups of the persistent grid;
    // split_hkv: tickets per item; split_min_cost: the least cost of an item
    // worth splitting.
    int split_cap, split_wgs, split_hkv, split_min_cost;
};

hipError_t launch_worklist(const WorklistArgs& a, hipStream_t stream);

// Operand modes of the attention kernels: token-block exponents; per-token
// exponents; per-token exponents with S from the E2M1 score views.
enum { MODE_BLOCK = 0, MODE_EXACT = 1, MODE_FP4 = 2 };

struct AttnArgs {
    int T, B, Hq, Hkv, causal;
    int mode;         // MODE_*
    int rotate;       // Q and K rotated (Hadamard): dQ and dK are rotated back
    int work_wgs;     // forward: workgroups of attention work (the rest write padding rows)
    float scale;      // softmax scale
    float c2;         // scale * log2(e)
    int scale_exp;    // f = floor(log2 scale)
    float scale_res;  // scale * 2^-f, in [1, 2)
    const int32_t* cu;
    const int32_t* count;
    const int32_t* items;
    int32_t* tickets;   // backward: the persistent grid's ticket counter (count + 1, zeroed with the list)
    // backward, 256-key tiles: count[2] leading items are split into two
    // tickets per kv head (halves of the iteration range); each half writes
    // its raw dK / dV accumulators to its slot of dkv_part (slots 2 p, 2 p + 1
    // of pair p = item x Hkv + kv head), which bwd_pair_kernel adds up
    float* dkv_part;
    const uint8_t *q_codes, *q_exps, *k_codes, *k_exps, *v_codes, *v_exps;
    // E2M1 score views (MODE_FP4): codes [T][H][D/2], E4M3 scales [T][H][D/16]
    const uint8_t *q_fp4, *q_fp4_scales, *k_fp4, *k_fp4_scales;
    // forward
    uint16_t* o;
    float* lse;
    // backward
    const float* lse_in;
    const uint8_t *do_codes, *do_exps;
    const float* delta;
    const int8_t* prescale;
    _Float16* dq_acc;
    uint16_t *dq, *dk, *dv;
    // optional: recorded just before / after the launch of the forward kernel
    // or of the backward main kernel
    hipEvent_t ev_start, ev_stop;
};

hipError_t launch_fwd(const AttnArgs& a, int D, int max_items, hipStream_t stream);
hipError_t launch_bwd(const AttnArgs& a, int D, int max_items, bool with_dq, hipStream_t stream);
// token-block operands only: 256-key tiles (work list built with tile 256)
hipError_t launch_bwd_wide(const AttnArgs& a, int D, int max_items, bool with_dq, hipStream_t stream);
hipError_t launch_bwd_dq(const AttnArgs& a, int D, int max_items, hipStream_t stream);
// workgroups of the persistent 256-key backward grid for up to `tickets` tickets
int bwd_wide_workgroups(int64_t tickets);
// dK / dV of the split pairs of the 256-key backward (after its main kernel)
hipError_t launch_bwd_pairs(const AttnArgs& a, int D, int max_pairs, hipStream_t stream);
hipError_t launch_bwd_finalize(const AttnArgs& a, int D, bool dq_from_acc, hipStream_t stream);

}  // namespace flamia
