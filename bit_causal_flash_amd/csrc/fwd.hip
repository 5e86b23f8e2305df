// fwd.hip -- causal packed microscaled attention forward for gfx950.
//
// Method (FLAMIA review section 2 "Why flash tiling recomputes scores",
// section 3 "Factoring the scales out of the score MMA", section 5
// Algorithm 1 steps 04-08 and "A range budget for probability
// quantization"; jaehun.me section 3.1):
//   S = Q^ K^T as an E4M3 MFMA on the stored codes, the Q and K token-block
//   exponents entering as per-row / per-column E8M0 operand scales (exact
//   powers of two); base-2 logits s2 = scale * log2(e) * S; an integer running
//   reference r = ceil(max s2); weights p = 2^(s2 - r) <= 1 boosted by 256
//   and rounded to E4M3 (the probability operand P^); l accumulates the
//   rounded weights; O += P^ V^ with V's per-32-key-block exponent and the
//   2^-8 un-boost as MFMA operand scales.  When r rises, O and l are
//   multiplied by the exact power of two 2^(r_old - r_new).
//   End: O = O / l (bf16), LSE = (r + log2 l) ln 2.
//
// Tiling: a workgroup (4 waves) owns one work-list item, a 128-query tile of
// one document and one q head; wave w owns 32 queries.  Keys are visited in
// document-relative 64-key steps staged in LDS, so every 32-key MFMA scale
// block is exactly one document-local token block.  S is computed transposed
// (S^T = K Q^T, lane = query) with the key rows permuted so that the
// accumulator layout already is the k layout the P^ V MFMA expects: P^ never
// leaves registers.  V is read k-major straight from its token-major LDS tile
// with ds_read_b64_tr_b8, so no transposed copy of V exists anywhere.  The
// next step's K/V tile is fetched into registers while the current one is
// processed (double-buffered LDS, one LDS-only barrier per step).  A few
// extra workgroups of the same launch write the rows after the last document.
#include "device.hpp"
#include "kernels.hpp"

namespace flamia {

namespace {

// One 64-key step of K and V, as staged for the forward through registers:
// D / 64 16-byte chunks per thread of the V codes and of the K codes
// (MODE_FP4: D / 8 bytes of the row's E2M1 K codes and the D / 64 scale bytes
// they use), and the raw exponents of key tid % 64 (K, and in the exact modes
// V) and of the V block of tid % 2.  At D = 128 the E4M3 codes bypass the
// registers (direct global -> LDS loads, see fwd_kernel) and only the rest
// comes through here.  Every load is unconditional, rows past the document
// end clamped to its last row (staging replaces their exponents, and the
// masks zero their weights), so that the only wait on the prefetch is where
// it is staged.
template <int D, int MODE>
struct KVTile {
    static constexpr int NC = D / 64;
    v4i k[NC], v[NC];
    v4i k4;
    uint32_t k4s;
    int ek, ev, evk, kok, vok;
};

template <int D, int MODE>
__device__ __forceinline__ void load_kvtile(const AttnArgs& a, KVTile<D, MODE>& r, int hk, int kt0,
                                            int e, int tid)
{
    constexpr int CPR = D / 16;
    const int Hkv = a.Hkv;
    const size_t T = (size_t)a.T;
    if constexpr (D != 128) {
#pragma unroll
        for (int k = 0; k < KVTile<D, MODE>::NC; ++k) {
            const int c = tid + 256 * k;
            const int row = c / CPR, col = 16 * (c % CPR);
            const int t = min(kt0 + row, e - 1);
            if constexpr (MODE != MODE_FP4)
                r.k[k] = *(const v4i*)(a.k_codes + ((size_t)t * Hkv + hk) * D + col);
            r.v[k] = *(const v4i*)(a.v_codes + ((size_t)t * Hkv + hk) * D + col);
        }
    }
    if constexpr (MODE == MODE_FP4) {
        // thread -> key row tid / 4, features (tid % 4) D / 4 .. + D / 4 - 1
        const int t = min(kt0 + (tid >> 2), e - 1);
        const int part = tid & 3;
        const uint8_t* src = a.k_fp4 + ((size_t)t * Hkv + hk) * (D / 2) + part * (D / 8);
        const uint8_t* ssrc = a.k_fp4_scales + ((size_t)t * Hkv + hk) * (D / 16) + part * (D / 64);
        if constexpr (D == 128) {
            r.k4 = *(const v4i*)src;
            r.k4s = (uint32_t)ssrc[0] | ((uint32_t)ssrc[1] << 8);
        } else {
            const v2i w = *(const v2i*)src;
            r.k4 = v4i{w.x, w.y, 0, 0};
            r.k4s = ssrc[0];
        }
    }
    if (kt0 + 64 <= e) {
        // a whole step inside the document (every step but a document's last):
        // a uniform base and the lane's offset, nothing to clamp
        const uint8_t* ke = a.k_exps + (size_t)hk * T + kt0;
        const uint8_t* ve = a.v_exps + (size_t)hk * T + kt0;
        r.kok = r.vok = 1;
        r.ek = ke[tid & 63];
        r.ev = ve[32 * (tid & 1)];
        if constexpr (MODE != MODE_BLOCK) r.evk = ve[tid & 63];
        return;
    }
    const int tk = kt0 + (tid & 63);
    const int tv = kt0 + 32 * (tid & 1);
    r.kok = tk < e;
    r.vok = tv < e;
    r.ek = a.k_exps[(size_t)hk * T + min(tk, e - 1)];
    r.ev = a.v_exps[(size_t)hk * T + min(tv, e - 1)];
    if constexpr (MODE != MODE_BLOCK) r.evk = a.v_exps[(size_t)hk * T + min(tk, e - 1)];
}

// Online-softmax update of one wave's 32 queries x 64 keys: the running
// integer reference r, and the probability operand P^ (byte 16 t + v <->
// key 32 t + 16 g + v) with its rounded row sum.  Unless `full`, element
// (t, v) is kept only if 32 t + v < lim.  With FOLD, the operand codes carry
// each key's V exponent relative to its 32-key block, vf[32 t + v] =
// 2^(e_V(j) - max e_V): P^ is rounded first (l sums the unshifted values),
// then shifted by that power of two, which is exact while the shifted weight
// stays in E4M3's normal range.
//
// The method rescales O and l by 2^(r_old - r_new) whenever r rises.  Here
// the accumulators instead stay in units of a per-query base R (the first
// finite reference): a step's P^ enters the O MFMA with the block scale
// 2^(r - R - 8) and its row sum is added to l with the same factor, so O and
// l hold exactly 2^(r - R) times the rescaled sums (a power of two commutes
// with every FP32 rounding), and the rescale is applied once, at the end.
// Only when r - R exceeds 32 are the accumulators rescaled and R moved up,
// which keeps them far from the FP32 range limit.  Returns the E8M0 code of
// the step's P^ scale.  (l stays a VALU sum: the MFMA's internal
// accumulation is not the exact FP32 sum of the rounded weights.)
template <int NDT, bool FOLD>
__device__ __forceinline__ int online_softmax(v16f (&sacc)[2], v16f (&oacc)[NDT], float& r,
                                              float& base, float& l, v8i& pf, float c2, bool full,
                                              int lim, const float* vf)
{
    if (!full) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (!(32 * t + v < lim)) sacc[t][v] = -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, sacc[t][v]);
    // the other half of the keys sits in the lane 32 away
    mloc = max_xor32(mloc);
    const float rn = fmaxf(r, ceilf(mloc * c2));
    r = rn;
    // nothing has been accumulated before the first finite reference
    if (base == -INFINITY) base = rn;
    if (__any(rn - base > 32.f)) {
        const bool mv = rn - base > 32.f;
        const float alpha = mv ? ldexpf(1.f, (int)fmaxf(base - rn, -200.f)) : 1.f;
        if (mv) base = rn;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    }
    const bool fin = rn != -INFINITY;
    const float off = fin ? 8.f - rn : 0.f;
    const int rel = fin ? (int)(rn - base) : 0;
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float p[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) p[k] = __builtin_amdgcn_exp2f(fmaf(sacc[t][4 * q + k], c2, off));
            const uint32_t w = cvt4_fp8(p[0], p[1], p[2], p[3]);
            lsum += sum4_fp8(w);
            if constexpr (FOLD) {
                const v4i fv = *(const v4i*)(vf + 32 * t + 4 * q);
                pf[4 * t + q] = (int)cvt4_fp8(p[0] * __int_as_float(fv.x), p[1] * __int_as_float(fv.y),
                                              p[2] * __int_as_float(fv.z), p[3] * __int_as_float(fv.w));
            } else {
                pf[4 * t + q] = (int)w;
            }
        }
    // the row sum is exact in FP32 (multiples of 2^-9 below 2^15), and so is
    // its product with the power of two
    l = fmaf(lsum, ldexpf(1.f, rel - 8), l);
    return kScaleMinus8 + rel;
}

// Modes: MODE_BLOCK token-block operands; MODE_EXACT per-token exponents (the
// V exponent folded into P^); MODE_FP4 the same with S from the E2M1 score
// views of Q and K, expanded to exact FP16 and contracted by the FP16 MFMA.
// Rows after the last document (t >= cu[B]): O = 0, LSE = +inf, written by
// kFwdPadWgs extra workgroups of the forward launch.
constexpr int kFwdPadWgs = 64;

template <int D>
__device__ void fwd_padding(const AttnArgs& a, int wg)
{
    const int ntok = a.cu[a.B];
    const size_t T = (size_t)a.T;
    const size_t first = (size_t)ntok * a.Hq * (D / 8);
    const size_t nchunks = T * a.Hq * (D / 8);
    for (size_t i = first + (size_t)wg * 256 + threadIdx.x; i < nchunks; i += (size_t)kFwdPadWgs * 256) {
        const size_t row = i / (D / 8);
        const int t = (int)(row / a.Hq), h = (int)(row % a.Hq);
        *(v4i*)(a.o + row * D + 8 * (i % (D / 8))) = v4i{0, 0, 0, 0};
        if (i % (D / 8) == 0) a.lse[(size_t)h * T + t] = INFINITY;
    }
}

// compile-time buffer index of a forward step
template <int V>
struct StepBuf {
    static constexpr int value = V;
};

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void fwd_kernel(AttnArgs a)
{
    if ((int)blockIdx.x >= a.work_wgs) {
        fwd_padding<D>(a, (int)blockIdx.x - a.work_wgs);
        return;
    }
    using CT = CodeTile<D>;            // K and V code tiles (swizzled rows at D = 128)
    constexpr int PITCH16 = 2 * D + 16;
    constexpr int NKS = D / 64;        // k steps over the head dim (E4M3 S)
    constexpr int NKH = D / 16;        // k steps over the head dim (FP16 S)
    constexpr int NDT = D / 32;        // 32-wide head-dim tiles of O
    constexpr int CPR = D / 16;        // 16-byte chunks per row
    constexpr bool FP4 = MODE == MODE_FP4;
    constexpr bool FOLD = MODE != MODE_BLOCK;
    // 128-byte aligned: at D = 128 the swizzled tiles are addressed by XOR
    __shared__ __attribute__((aligned(128))) uint8_t s_k[2][FP4 ? 64 * PITCH16 : 64 * CT::PITCH];
    __shared__ __attribute__((aligned(128))) uint8_t s_v[2][64 * CT::PITCH];
    __shared__ int s_ek[2][64];
    __shared__ int s_ev[2][2];
    __shared__ __attribute__((aligned(16))) float s_vf[2][FOLD ? 64 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), g = lane >> 5;
    const int Hq = a.Hq, Hkv = a.Hkv;
    const size_t T = (size_t)a.T;
    // consecutive workgroups cycle over the kv heads first, so that the q
    // heads sharing a kv head land on the same XCD (workgroup i runs on XCD
    // i % 8) and share its L2 copy of the K/V tiles
    const int item = blockIdx.x / Hq, rr = blockIdx.x % Hq;
    const int h = (rr % Hkv) * (Hq / Hkv) + rr / Hkv;
    if (item >= *a.count) return;
    const int b = a.items[2 * item], m = a.items[2 * item + 1];
    const int s = a.cu[b], e = a.cu[b + 1];
    const int hk = h * Hkv / Hq;
    const int q0 = s + 128 * m;
    const int qw = q0 + 32 * wave;
    const int qi = qw + (lane & 31);
    const bool qvalid = qi < e;
    const float c2 = a.c2;

    // Q fragments: B operand of S^T = K Q^T (lane = query column, k = head
    // dim): E4M3 codes with the query's exponent, or the FP16 expansion of
    // its E2M1 view (k = 16 per FP16 step: features 16 ks + 8 g .. + 7)
    v8i qf[FP4 ? 1 : NKS];
    h8 qh[FP4 ? NKH : 1];
    int eq = 127;
    if constexpr (FP4) {
        const size_t row = (size_t)min(qi, e - 1) * Hq + h;
#pragma unroll
        for (int ks = 0; ks < NKH; ++ks) {
            const uint32_t c = *(const uint32_t*)(a.q_fp4 + row * (D / 2) + 8 * ks + 4 * g);
            const float sc = __builtin_amdgcn_cvt_f32_fp8((int)a.q_fp4_scales[row * (D / 16) + ks], 0);
            qh[ks] = fp4x8_to_f16(c, sc);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (qvalid) qf[ks] = row_operand(a.q_codes + ((size_t)qi * Hq + h) * D + 64 * ks, lane);
            else qf[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
        eq = qvalid ? (int)a.q_exps[(size_t)h * T + qi] : 127;
    }

    const int kend = a.causal ? min(q0 + 128, e) : e;
    const int nsteps = (kend - s + 63) / 64;
    // keys the wave's queries can see; none when all of its queries lie past
    // the document end (the last tile of a document): such a wave only
    // helps stage the K/V tiles
    const int kend_w = qw >= e ? s : (a.causal ? min(qw + 32, e) : e);

    v16f oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
    float r = -INFINITY;     // integer base-2 row reference
    float base = -INFINITY;  // reference the accumulators are kept in
    float l = 0.f;           // sum of rounded weights

    // D = 128: the E4M3 code tiles go from global memory straight into the
    // swizzled LDS layout.  Wave w fills rows 16 w .. 16 w + 15 of each tile
    // with two loads of 1 KB (eight rows), lane L of a load writing LDS bytes
    // 16 L .. 16 L + 15 of its block: row + L / 8, physical chunk L % 8, so it
    // fetches the logical chunk (L % 8) ^ tile_swizzle(row).
    constexpr bool DMA = CT::SWZ;
    // the lane's byte offsets of its two rows from the step's first row
    uint32_t dma_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * wave + 8 * i + (lane >> 3);
        dma_off[i] = (uint32_t)(row * Hkv * D + 16 * ((lane & 7) ^ tile_swizzle(row)));
    }
    auto dma = [&](int kt0, int buf) {
        if constexpr (DMA) {
            if (kt0 + 64 <= e) {
                // every row inside the document: a uniform base plus the offsets
                const size_t base = ((size_t)kt0 * Hkv + hk) * D;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int rb = 16 * wave + 8 * i;
                    if constexpr (!FP4) dma16_opaque_s(a.k_codes + base, dma_off[i], (lds_void*)&s_k[buf][rb * 128]);
                    dma16_opaque_s(a.v_codes + base, dma_off[i], (lds_void*)&s_v[buf][rb * 128]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int rb = 16 * wave + 8 * i;
                    const int row = rb + (lane >> 3);
                    const int c = (lane & 7) ^ tile_swizzle(row);
                    const size_t src = ((size_t)min(kt0 + row, e - 1) * Hkv + hk) * D + 16 * c;
                    if constexpr (!FP4) dma16_opaque(a.k_codes + src, (lds_void*)&s_k[buf][rb * 128]);
                    dma16_opaque(a.v_codes + src, (lds_void*)&s_v[buf][rb * 128]);
                }
            }
        }
    };

    // every thread writes (the four waves write identical exponents), so
    // that every prefetched register is consumed on every path
    auto stage = [&](const KVTile<D, MODE>& t, int buf) {
        if constexpr (!DMA) {
#pragma unroll
            for (int k = 0; k < KVTile<D, MODE>::NC; ++k) {
                const int c = tid + 256 * k;
                const int row = c / CPR, col = 16 * (c % CPR);
                if constexpr (!FP4) *(v4i*)(&s_k[buf][CT::off(row, col)]) = t.k[k];
                *(v4i*)(&s_v[buf][CT::off(row, col)]) = t.v[k];
            }
        }
        if constexpr (FP4) {
            // the row's features (tid % 4) D / 4 .. + D / 4 - 1 as FP16
            uint8_t* dst = &s_k[buf][(tid >> 2) * PITCH16 + 2 * (tid & 3) * (D / 4)];
#pragma unroll
            for (int q = 0; q < D / 32; ++q) {
                const float sc = __builtin_amdgcn_cvt_f32_fp8((int)((t.k4s >> (8 * (q / 2))) & 0xff), 0);
                *(h8*)(dst + 16 * q) = fp4x8_to_f16((uint32_t)t.k4[q], sc);
            }
        }
        s_ek[buf][tid & 63] = t.kok ? t.ek : 127;
        if constexpr (FOLD) {
            // lane = key: the V block exponent is the largest over the
            // block's valid keys, and the key's fold factor its offset
            const uint32_t ek = t.kok ? (uint32_t)t.evk : 0u;
            const uint32_t emax = half_wave_max_u32(ek);
            s_ev[buf][(tid & 63) >> 5] = (int)emax;
            s_vf[buf][tid & 63] = t.kok ? ldexpf(1.f, (int)ek - (int)emax) : 0.f;
        } else {
            s_ev[buf][tid & 1] = t.vok ? t.ev : 127;
        }
    };

    KVTile<D, MODE> nxt;
    load_kvtile<D, MODE>(a, nxt, hk, s, e, tid);
    dma(s, 0);
    stage(nxt, 0);
    // every load issued so far has landed (vmcnt(0)), so that inside the loop
    // only the prefetch of the next step is outstanding; the builtin wait
    // (free after the asm one) tells the compiler that the Q fragments have
    // landed, so it puts no wait for them inside the loop
    if constexpr (DMA) wait_vm0_asm();
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();

    // One 64-key step; the buffer index is a compile-time constant (the loop
    // below takes two steps per trip), so every LDS operand address is a
    // loop-invariant lane base plus an immediate offset.
    auto step = [&](int st, auto cur_c) __attribute__((always_inline)) {
        constexpr int cur = decltype(cur_c)::value;
        const int kt0 = s + 64 * st;
        // prefetch the next step (the last step reloads its own, unused)
        const int kn0 = min(kt0 + 64, s + 64 * (nsteps - 1));
        load_kvtile<D, MODE>(a, nxt, hk, kn0, e, tid);
        dma(kn0, cur ^ 1);
        const uint8_t* sk = s_k[cur];
        const uint8_t* sv = s_v[cur];

        if (kt0 < kend_w) {
            // S^T tiles: tile t row rho <-> key perm_row(t, rho) of the step
            v16f sacc[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int krow = perm_row(t, lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) sacc[t][v] = 0.f;
                if constexpr (FP4) {
#pragma unroll
                    for (int ks = 0; ks < NKH; ++ks)
                        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            *(const h8*)(sk + krow * PITCH16 + 2 * (16 * ks + 8 * g)), qh[ks], sacc[t],
                            0, 0, 0);
                } else {
                    const int ek = s_ek[cur][krow];
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        sacc[t] = mfma_f8(CT::SWZ ? swz_row_operand(swz_row_addr(s_k[0], krow, lane), ks,
                                                                    cur * (int)sizeof(s_k[0]))
                                                  : tile_row_operand<D>(sk, krow, 64 * ks, lane),
                                          qf[ks],
                                          sacc[t], ek, eq);
                }
            }

            // masking is needed only where the step runs past the document
            // end or, causally, some key follows some query of the wave;
            // element (t, v) is key kt0 + 32 t + 16 g + v
            v8i pf;
            const bool full = (kt0 + 64 <= e) && (!a.causal || kt0 + 63 <= qw);
            const int lim = min(e, a.causal ? qi + 1 : e) - kt0 - 16 * g;
            const int sp = online_softmax<NDT, FOLD>(sacc, oacc, r, base, l, pf, c2, full, lim,
                                                     FOLD ? &s_vf[cur][16 * g] : nullptr);

            // O^T += V^T P^T: V^T read k-major from the token-major LDS tile
            const int sv_exp = s_ev[cur][g];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                oacc[dt] = mfma_f8(CT::SWZ ? swz_tr_operand(swz_tr_addr(s_v[0], lane), 0, dt, cur * (int)sizeof(s_v[0]))
                                           : tile_tr_operand<D>(sv, 0, 32 * dt, lane),
                                   pf, oacc[dt],
                                   sv_exp, sp);
        }
        stage(nxt, cur ^ 1);
        // the direct loads count in vmcnt: they have landed once it is zero
        // (a wait the compiler cannot drop: it does not see the asm loads)
        if constexpr (DMA) wait_vm0_asm();
        lds_barrier();
    };
    for (int st = 0; st < nsteps; st += 2) {
        step(st, StepBuf<0>{});
        if (st + 1 < nsteps) step(st + 1, StepBuf<1>{});
    }

    l = sum_xor32(l);
    if (qvalid) {
        // O / l needs no rescale (both carry 2^(r - base)); the LSE takes the
        // rescaled sum
        const float inv = 1.f / l;
        l = ldexpf(l, (int)(base - r));
        uint16_t* orow = a.o + ((size_t)qi * Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v2i w;
                w.x = (int)pack_bf16x2(oacc[dt][4 * q] * inv, oacc[dt][4 * q + 1] * inv);
                w.y = (int)pack_bf16x2(oacc[dt][4 * q + 2] * inv, oacc[dt][4 * q + 3] * inv);
                *(v2i*)(orow + 32 * dt + 8 * q + 4 * g) = w;
            }
        if (g == 0) a.lse[(size_t)h * T + qi] = (r + __log2f(l)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd(const AttnArgs& a, int D, int max_items, hipStream_t stream)
{
    if (max_items <= 0) return hipSuccess;
    AttnArgs args = a;
    args.work_wgs = max_items * a.Hq;
    const dim3 grid((unsigned)(args.work_wgs + kFwdPadWgs));
#define FLAMIA_FWD(DD, MM) \
    FLAMIA_LAUNCH((fwd_kernel<DD, MM>), grid, dim3(256), stream, args.ev_start, args.ev_stop, args)
    if (D == 128) {
        if (a.mode == MODE_FP4) FLAMIA_FWD(128, MODE_FP4);
        else if (a.mode == MODE_EXACT) FLAMIA_FWD(128, MODE_EXACT);
        else FLAMIA_FWD(128, MODE_BLOCK);
    } else {
        if (a.mode == MODE_FP4) FLAMIA_FWD(64, MODE_FP4);
        else if (a.mode == MODE_EXACT) FLAMIA_FWD(64, MODE_EXACT);
        else FLAMIA_FWD(64, MODE_BLOCK);
    }
#undef FLAMIA_FWD
    return hipGetLastError();
}

}  // namespace flamia
