/*
 * flamia.h -- C ABI of the MI355X (gfx950) causal packed microscaled attention
 * library: document-local token-block E4M3 quantization, the online-softmax
 * forward and the recomputed backward of the FLAMIA method.
 *
 * Method references (pages and sections):
 *   "FLAMIA ... technical review" (zhongzhuzhou.org, 2026-11-08):
 *     section 2 "Prerequisites" (attention, backward products, D identity,
 *     online softmax), section 3 "Reusable scales and score formation"
 *     (document-local 32-token blocks x full head dim, separable score
 *     scaling), section 4 "A causal mask must include scale selection"
 *     (conservative exponent, causal dQ accumulator scale), section 5
 *     Algorithm 1 and "A range budget for probability quantization",
 *     section 6 "Packed documents and GPU scheduling" and Algorithm 2.
 *   jaehun.me review of arXiv 2611.03344, sections 3.1-3.4 (E4M3 token
 *     blocks for Q, K, V, dO; one scale per 32x32 dS block; FP16 dQ
 *     partials with a power-of-two prescale; BF16 outputs).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates device memory, never synchronises and never
 *     reads device memory on the host: every call is asynchronous on
 *     `stream` (a hipStream_t; NULL is the default stream) and consists only
 *     of kernel launches.
 *   - Errors are returned as status codes, never raised.  Host-side arguments
 *     are validated before any launch; FLAMIA_ERR_HIP reports a launch
 *     failure (hipGetLastError).  Device-side preconditions on cu_seqlens are
 *     documented, not checked: violating them is undefined behaviour.
 *   - Layouts (row-major, packed along tokens):
 *       bf16 activations   uint16 [T][H][d]
 *       E4M3 codes         uint8  [T][H][d]     (OCP E4M3FN)
 *       exponent tables    uint8  [H][T]        (UE8M0 byte e + 127, one per
 *                                                token, replicated over its
 *                                                block)
 *       LSE                float  [Hq][T]       (natural log)
 *   - Rows t >= cu_seqlens[B] are padding: codes 0, exponent byte 127,
 *     O = 0, LSE = +inf, dQ = dK = dV = 0.
 *   - GQA: q head h reads kv head floor(h * Hkv / Hq) (contiguous groups).
 *   - Thread-safety: no global mutable state (except the fixed scratch array
 *     of flamia_attn_fwd_noalloc, described there); concurrent calls on
 *     different streams with disjoint outputs and workspaces are safe.
 */
#ifndef FLAMIA_H
#define FLAMIA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FLAMIA_OK = 0,
    FLAMIA_ERR_INVALID_ARG = 1, /* a host-side argument is out of range or NULL */
    FLAMIA_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim 96) */
    FLAMIA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required */
    FLAMIA_ERR_HIP = 4          /* a kernel launch failed */
} flamia_status;

/* Problem flags. */
enum {
    FLAMIA_CAUSAL = 1u << 0,        /* keys j <= i of the query's document */
    FLAMIA_EXACT = 1u << 1,         /* exact-scale option: operands quantized
                                       with FLAMIA_SCALE_PER_TOKEN, per-token dO,
                                       per-(query row, 32-key block) dS
                                       exponents for dQ; not with
                                       FLAMIA_DETERMINISTIC in the backward */
    FLAMIA_FP4_SCORE = 1u << 2,     /* scores from the E2M1 views of Q and K
                                       (FLAMIA_SCALE_NVFP4_16); requires
                                       FLAMIA_EXACT; backward: head_dim 64 */
    FLAMIA_DETERMINISTIC = 1u << 3, /* bitwise run-to-run repeatable backward */
    FLAMIA_HADAMARD = 1u << 4,      /* Q and K codes come from the rotated rows
                                       (FLAMIA_SCALE_ROTATE); not with
                                       FLAMIA_EXACT, nor with
                                       FLAMIA_DETERMINISTIC in the backward */
    FLAMIA_DQ_PRESCALE_SEQUENCE = 1u << 5 /* test-only negative control, backward
                                       only: the dQ prescale from sequence-wide
                                       maxima instead of each row's visible
                                       keys (a later outlier then moves the
                                       FP16 rounding of earlier rows); not with
                                       FLAMIA_DETERMINISTIC */
};

/* Quantizer scale policies. */
enum {
    FLAMIA_SCALE_TOKBLOCK32 = 0, /* one exponent per document-local block of
                                    <= 32 tokens x full head dim */
    FLAMIA_SCALE_PER_TOKEN = 1,  /* one exponent per token x full head dim */
    FLAMIA_SCALE_NVFP4_16 = 2,   /* score view: E2M1 codes + an E4M3 scale per
                                    16 in-token features */
    FLAMIA_SCALE_ROTATE = 0x100, /* OR-ed into TOKBLOCK32 or PER_TOKEN: rotate
                                    every row by the Hadamard matrix first */
    FLAMIA_SCALE_FLOOR_CONTROL = 0x200 /* OR-ed into TOKBLOCK32 or PER_TOKEN:
                                    the reference floor exponent rule
                                    e = floor(log2 amax) - 8 with saturation
                                    at 448 (jaehun.me section 2), which can
                                    leak a later token of a block into an
                                    earlier one's value.  A negative control
                                    for causality tests only. */
};

/* Optional timing hook: hipEvent_t handles that the library records on the
 * call's stream just before and just after the launch of the quantizer
 * kernel of flamia_quantize_tokblock and flamia_quantize_qkv, the forward
 * kernel of flamia_attn_fwd or the backward main kernel of flamia_attn_bwd,
 * so that their elapsed time is that kernel's.  The launch is the same with
 * or without them.  Either may be NULL.  The caller owns the events. */
typedef struct {
    void* attn_start;
    void* attn_stop;
} flamia_kernel_events;

typedef struct {
    int32_t total_tokens;       /* T >= 0: rows of every packed buffer */
    int32_t num_seqs;           /* B >= 1 */
    const int32_t* cu_seqlens;  /* DEVICE int32 [B + 1]; cu[0] = 0, nondecreasing,
                                   cu[B] <= T (unchecked: UB if violated) */
    int32_t num_q_heads;        /* Hq >= 1 */
    int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t head_dim;           /* d in {64, 128} */
    float softmax_scale;        /* <= 0 selects 1 / sqrt(d) */
    uint32_t flags;             /* FLAMIA_* flags */
    const flamia_kernel_events* events; /* optional timing events, or NULL */
} flamia_problem;

/*
 * Token-block quantizer (review section 3 "Why one shared exponent can serve
 * two reductions"; section 4 conservative exponent; jaehun.me section 3.1).
 * With FLAMIA_SCALE_NVFP4_16 it instead writes the E2M1 score view of
 * review section 2 / jaehun.me section 3.1 (no tensor-level scale): for each
 * (token, head, group of 16 features), s = the smallest E4M3 value with
 * amax / s <= 6 (s = 1 for a zero group), codes = nearest E2M1 value of x / s
 * with ties to the even code (sign in bit 3);
 *     codes [T][H][d / 2] (feature 2k in the low nibble of byte k),
 *     exps  [T][H][d / 16] (the E4M3 scale bytes);
 * padding rows get zero codes and scale 1.0 (0x38).
 * For each head and each document-local block of up to 32 consecutive tokens
 * (blocks start at every document start; the last may be partial), with amax
 * the block's largest |x| over all d features:
 *     e = smallest integer with amax / 2^e <= 448   (e = 0 for amax = 0),
 *         clamped to [-127, 127];
 *     codes = E4M3(x * 2^-e), nearest with ties to even;
 *     exps[h][t] = e + 127 on every token of the block.
 *   p          problem; only total_tokens, num_seqs and cu_seqlens are read
 *   num_heads  H >= 1 of this tensor (Hq for Q, Hkv for K and V)
 *   scale_mode FLAMIA_SCALE_TOKBLOCK32, FLAMIA_SCALE_PER_TOKEN or
 *              FLAMIA_SCALE_NVFP4_16; the first two may be OR-ed with
 *              FLAMIA_SCALE_ROTATE (review section 3 "Rotation, range, and
 *              the alternative", Algorithm 1 step 02; jaehun.me section 3.4):
 *              every row x (d features) is first replaced by x H_d, H_d the
 *              Sylvester Hadamard matrix (entries (-1)^popcount(i & j),
 *              H_d H_d = d I), computed in FP32 by the fast Walsh-Hadamard
 *              transform (butterflies (a, b) -> (a + b, a - b) for pair
 *              distances 1, 2, ..., d / 2 in that order); the block maxima and
 *              codes are those of the rotated values.  For Q and K of a
 *              FLAMIA_HADAMARD problem.
 *   x          bf16 [T][H][d] (device, read)
 *   codes      uint8 [T][H][d] (device, written)
 *   exps       uint8 [H][T] (device, written)
 * Returns FLAMIA_ERR_UNSUPPORTED when ceil(T / 32) * H >= 2^24 (one
 * 256-thread workgroup per 32-token window and head); the attention calls
 * apply the same limit to Hq.
 */
flamia_status flamia_quantize_tokblock(const flamia_problem* p, int32_t num_heads,
                                       int32_t scale_mode, const uint16_t* x, uint8_t* codes,
                                       uint8_t* exps, void* stream);

/*
 * Q, K and V of one problem in a single launch: the same results as
 * flamia_quantize_tokblock on each (num_heads = num_q_heads for Q,
 * num_kv_heads for K and V), with FLAMIA_SCALE_ROTATE in scale_mode
 * applying to Q and K only and FLAMIA_SCALE_FLOOR_CONTROL to all three.
 *   scale_mode FLAMIA_SCALE_TOKBLOCK32 or FLAMIA_SCALE_PER_TOKEN, optionally
 *              OR-ed with FLAMIA_SCALE_ROTATE / FLAMIA_SCALE_FLOOR_CONTROL
 *   q, k, v    bf16 [T][Hq][d], [T][Hkv][d], [T][Hkv][d] (device, read)
 *   *_codes    uint8 like their inputs; *_exps uint8 [H][T] (device, written)
 * Returns FLAMIA_ERR_INVALID_ARG for NULL pointers (T > 0) or another scale
 * mode, FLAMIA_ERR_UNSUPPORTED when ceil(T / 32) * (Hq + 2 Hkv) >= 2^24.
 */
flamia_status flamia_quantize_qkv(const flamia_problem* p, int32_t scale_mode, const uint16_t* q,
                                  const uint16_t* k, const uint16_t* v, uint8_t* q_codes,
                                  uint8_t* q_exps, uint8_t* k_codes, uint8_t* k_exps,
                                  uint8_t* v_codes, uint8_t* v_exps, void* stream);

/*
 * Forward (review section 2 online softmax, section 3 separable score
 * scaling, section 5 Algorithm 1 steps 04-08 and the range budget):
 *   s2_ij = softmax_scale * log2(e) * Q^_i . K^_j over visible keys, with the
 *   Q/K token-block exponents applied as row and column factors;
 *   per row an integer base-2 reference r = ceil(max s2) (running), weights
 *   p = 2^(s2 - r), probability operand P^ = E4M3(256 p) / 256,
 *   l = sum P^, O = sum P^ V^ / l (bf16), LSE = (r + log2 l) ln 2.
 * Inputs are the quantizer's outputs for Q (Hq heads), K and V (Hkv heads).
 *   o          bf16 [T][Hq][d] (written)
 *   lse        float [Hq][T] (written)
 *   workspace  device scratch of at least flamia_attn_fwd_workspace_size(p)
 *              bytes; its contents are overwritten.
 * With FLAMIA_EXACT the Q/K/V exponents are per token and enter the score
 * and dP products through the matrix cores' per-row/per-column scales; the
 * V exponent, which varies along the P^ V contraction, is folded into P^
 * (its FP32 value times 2^(e_V(j) - max over the 32-key block) before the
 * E4M3 rounding, equal to the unfolded product in E4M3's normal range); l
 * still sums the unfolded P^.  With FLAMIA_FP4_SCORE s2 is computed from the
 * E2M1 views (q_fp4 / k_fp4: codes uint8 [T][H][d/2], scales uint8
 * [T][H][d/16], as FLAMIA_SCALE_NVFP4_16 writes them); the fp4 pointers must
 * be NULL without the flag and non-NULL with it.
 * With FLAMIA_HADAMARD the Q and K codes must be those of the rotated rows
 * (FLAMIA_SCALE_ROTATE): since q H . k H = d q . k, the softmax scale is
 * divided by d, and O and LSE are those of the unrotated problem up to
 * rounding.
 */
size_t flamia_attn_fwd_workspace_size(const flamia_problem* p);
flamia_status flamia_attn_fwd(const flamia_problem* p, const uint8_t* q_codes,
                              const uint8_t* q_exps, const uint8_t* k_codes,
                              const uint8_t* k_exps, const uint8_t* v_codes,
                              const uint8_t* v_exps, const uint8_t* q_fp4,
                              const uint8_t* q_fp4_scales, const uint8_t* k_fp4,
                              const uint8_t* k_fp4_scales, uint16_t* o, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and results as flamia_attn_fwd, with the work list in
 * a fixed device array of the library instead of a caller's workspace.
 *   - The array holds flamia_attn_fwd_noalloc_scratch_bytes() bytes (4 MiB):
 *     a problem whose forward workspace (flamia_attn_fwd_workspace_size)
 *     exceeds it returns FLAMIA_ERR_WORKSPACE before any launch.  4 MiB
 *     covers, for instance, any document count up to 2^18 tokens, or up to
 *     2^20 tokens in at most 2^16 documents.
 *   - Each GPU the library runs on holds its own array until the process
 *     ends; the call uses the one of the current device, so `stream` must
 *     belong to it.  The array's device address is looked up on the first
 *     call on each device (no allocation; make that first call outside a
 *     graph capture).
 *   - Every call on a GPU shares that GPU's array and leaves it holding the
 *     last call's work list: calls that overlap on one GPU (several streams,
 *     or several threads) race and must be ordered by the caller.
 *   - Nothing is allocated or freed; the other arguments are as for
 *     flamia_attn_fwd.
 */
size_t flamia_attn_fwd_noalloc_scratch_bytes(void);
flamia_status flamia_attn_fwd_noalloc(const flamia_problem* p, const uint8_t* q_codes,
                                      const uint8_t* q_exps, const uint8_t* k_codes,
                                      const uint8_t* k_exps, const uint8_t* v_codes,
                                      const uint8_t* v_exps, const uint8_t* q_fp4,
                                      const uint8_t* q_fp4_scales, const uint8_t* k_fp4,
                                      const uint8_t* k_fp4_scales, uint16_t* o, float* lse,
                                      void* stream);

/*
 * Backward (review section 5 Algorithm 1 steps 09-16; jaehun.me sections
 * 3.1-3.4).  dO is quantized inside the call with the operand rule;
 * D_i = dO^_i . O_i; P is rebuilt from the saved LSE; dP = dO^ V^T;
 * dS = P (dP - D); P^ = E4M3(256 P) / 256; dS is quantized with one
 * conservative exponent per document-local 32x32 block;
 *   dV = P^T dO^,  dK = scale dS^T Q^,  dQ = scale dS^ K^.
 * dQ partials are accumulated in FP16 after a per-row power-of-two prescale
 * 2^k_i that depends only on what row i may see (k_i = 14 - C - (e_dO(i) +
 * max visible V exponent + max visible K exponent), C = ceil(log2(4 scale d
 * 448^3))), and unscaled at the end; with FLAMIA_DETERMINISTIC dQ is instead
 * accumulated in FP32 registers by query-major blocks, so repeated calls are
 * bitwise identical.  dK and dV sum over the q heads of each kv group.
 *   o, lse     the forward's outputs
 *   dout       bf16 [T][Hq][d]
 *   dq         bf16 [T][Hq][d] (written)
 *   dk, dv     bf16 [T][Hkv][d] (written)
 *   workspace  at least flamia_attn_bwd_workspace_size(p) bytes; it holds the
 *              quantized dO, D, k_i, the FP16 dQ accumulator and work lists,
 *              at the offsets flamia_attn_bwd_workspace_layout reports, and
 *              (at most 64 MB) FP32 dK / dV halves of work items the call
 *              splits in two when they are few and long; the halves are added
 *              in a fixed order, so repeated calls give identical dK and dV.
 * FLAMIA_HADAMARD: Q and K codes of the rotated rows; the gradient products
 * use them at softmax scale / d, and dQ, dK are taken back to the original
 * coordinates (times H_d) before they are written.
 * FLAMIA_DQ_PRESCALE_SEQUENCE (test-only negative control; review section 4
 * "Forward locality and backward locality differ", jaehun.me section 3.3):
 * every row of q head h takes k = 14 - C - (max e_dO + max e_V + max e_K),
 * the maxima over all tokens of all documents (h for dO, its kv head for V
 * and K), clamped to [-60, 60]; padding rows 0.  Only the FP16 rounding of dQ
 * changes.  Returns FLAMIA_ERR_UNSUPPORTED with FLAMIA_DETERMINISTIC, whose
 * FP32 dQ has no prescale.
 * FLAMIA_EXACT (review section 4; jaehun.me section 3.2): dO is quantized per
 * token; the dO, Q and K exponents, which vary along the contractions of
 * dV, dK and dQ, are folded into P^, dS^ (dK copy) and dS^ (dQ copy) before
 * their E4M3 rounding; the dQ copy of dS carries one exponent per (query
 * row, 32-key block), from the row's largest |dS| over that block.  Returns
 * FLAMIA_ERR_UNSUPPORTED with FLAMIA_DETERMINISTIC, and with
 * FLAMIA_FP4_SCORE at head_dim 128.
 */
size_t flamia_attn_bwd_workspace_size(const flamia_problem* p);
flamia_status flamia_attn_bwd(const flamia_problem* p, const uint8_t* q_codes,
                              const uint8_t* q_exps, const uint8_t* k_codes,
                              const uint8_t* k_exps, const uint8_t* v_codes,
                              const uint8_t* v_exps, const uint8_t* q_fp4,
                              const uint8_t* q_fp4_scales, const uint8_t* k_fp4,
                              const uint8_t* k_fp4_scales, const uint16_t* o, const float* lse,
                              const uint16_t* dout, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Byte offsets, inside the backward workspace, of what a backward call left
 * there: dO codes uint8 [T][Hq][d], dO exponents uint8 [Hq][T], D float
 * [Hq][T], prescale exponents int8 [Hq][T] and the FP16 dQ accumulator
 * [T][Hq][d] (scaled by 2^k_i).  Returns FLAMIA_ERR_INVALID_ARG for an
 * invalid problem. */
typedef struct {
    size_t do_codes, do_exps, delta, dq_prescale, dq_accum, total;
} flamia_bwd_workspace_layout;
flamia_status flamia_attn_bwd_workspace_layout(const flamia_problem* p,
                                               flamia_bwd_workspace_layout* out);

/* Static string for a status code. */
const char* flamia_status_string(flamia_status s);

#ifdef __cplusplus
}
#endif

#endif /* FLAMIA_H */
