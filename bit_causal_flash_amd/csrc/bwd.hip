// bwd.hip -- causal packed microscaled attention backward for gfx950.
//
// Method (FLAMIA review section 2 "The contraction moves between forward and
// backward" and "The softmax gradient is a centered product", section 4
// "Forward locality and backward locality differ", section 5 Algorithm 1
// steps 11-16; jaehun.me sections 3.1-3.4):
//   P  = 2^(s2 - LSE log2 e) rebuilt from the saved LSE with the forward's
//        score path (same codes, same separable exponents);
//   dP = dO^ V^T, dS = P (dP - D);
//   P^ = E4M3(256 P) (un-boosted by 2^-8 inside the MFMA);
//   dS^ = E4M3 codes with one conservative exponent per document-local
//        32 x 32 block (its largest |dS| over visible entries);
//   dV += P^T dO^,  dK += dS^T Q^ (times scale at the end),
//   dQ partial = scale dS^ K^, multiplied by the row's prescale 2^k_i and
//        added into an FP16 accumulator with packed atomics; the finalize
//        kernel divides the prescale back out and writes bf16.
//
// Tiling: a workgroup owns a document-local 128-key tile of one kv head and
// loops over the q heads of its group and the 64-query tiles that can see its
// keys.  Its 8 waves have two roles (see bwd_kernel): score waves (S, dP, P,
// dS for one 32-key token block each) and gradient waves (dV, dK for the same
// keys, accumulated in registers across the whole loop, i.e. the GQA head
// reduction without atomics, and the tile's dQ).  S and dP are computed with
// the query rows permuted so the accumulators already hold P^ and dS^ in the
// k layout of the dV / dK MFMAs.  Q, dO and K are staged token-major in LDS
// and read k-major with ds_read_b64_tr_b8 where the contraction runs over
// tokens: one copy of every code tensor serves both orientations.  dS^ goes
// through LDS once, key-major, and is read transposed for dQ.  Barriers order
// LDS traffic only.  The dQ partials (one per query tile and 128-key tile)
// are added with packed FP16 atomics, whose throughput, not the MFMAs, bounds
// the kernel on long documents.
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"

namespace flamia {

namespace {

// One 64-query tile of one q head, as staged for the backward by NT threads:
// 8 D / NT 16-byte chunks per thread of the Q and dO code tiles (chunk
// c < 4 D of Q, the rest of dO) and the raw per-query values of row tid % 64.
// Every load is unconditional, with rows past the document end clamped to
// its last row (their statistics are replaced at staging, which makes their
// P, and so their dS, exactly zero), so that the only wait on the prefetch
// is where it is staged.
template <int D, int NT>
struct QTile {
    static constexpr int NC = 8 * D / NT;
    v4i c[NC];
    int eq, edo, pre, ok;
    float lse, delta;
    // E2M1 view of the Q rows (MODE_FP4): row tid / 4, D / 8 code bytes and
    // D / 64 scale bytes from feature (tid % 4) D / 4
    v2i q4;
    uint32_t q4s;
};

template <int D, int NT, int MODE>
__device__ __forceinline__ void load_qtile(const AttnArgs& a, QTile<D, NT>& r, int h, int qb, int e,
                                           int tid)
{
    if constexpr (MODE == MODE_FP4) {
        const size_t row = (size_t)min(qb + (tid >> 2), e - 1) * a.Hq + h;
        r.q4 = *(const v2i*)(a.q_fp4 + row * (D / 2) + (tid & 3) * (D / 8));
        r.q4s = a.q_fp4_scales[row * (D / 16) + (tid & 3) * (D / 64)];
    }
    constexpr int CPR = D / 16;
    const int Hq = a.Hq;
    const size_t T = (size_t)a.T;
#pragma unroll
    for (int k = 0; k < QTile<D, NT>::NC; ++k) {
        const int c = tid + NT * k;
        const bool isq = c < 4 * D;
        const int cc = isq ? c : c - 4 * D;
        const int row = cc / CPR, col = 16 * (cc % CPR);
        const int t = min(qb + row, e - 1);
        const uint8_t* src = isq ? a.q_codes : a.do_codes;
        r.c[k] = *(const v4i*)(src + ((size_t)t * Hq + h) * D + col);
    }
    const int t = qb + (tid & 63);
    r.ok = t < e;
    const size_t i = (size_t)h * T + min(t, e - 1);
    r.eq = a.q_exps[i];
    r.edo = a.do_exps[i];
    r.lse = a.lse_in[i];
    r.delta = a.delta[i];
    r.pre = a.prescale[i];
}

// 256 P and 256 dS of one wave's 32 keys x 32 queries, in place, and the
// largest |256 dS|.  Element v of lane group g is query 16 g + v of the
// wave's 32 (the statistics nl, dl start at that query); with MASK it is
// kept only if v >= lim (causal visibility and key validity folded into lim).
template <bool MASK>
__device__ __forceinline__ float softmax_grad(v16f& sacc, v16f& pacc, const float* nl,
                                              const float* dl, float c2, int lim)
{
    float amax = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[v], c2, nl[v]));
        if (MASK) p = (v >= lim) ? p : 0.f;
        const float ds = p * (pacc[v] - dl[v]);
        sacc[v] = p;
        pacc[v] = ds;
        amax = fmaxf(amax, fabsf(ds));
    }
    return amax;
}

// The same with pacc already holding dP - D (the dP product accumulated
// onto -D).
template <bool MASK>
__device__ __forceinline__ float softmax_grad_c(v16f& sacc, v16f& pacc, const float* nl, float c2, int lim)
{
    float amax = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[v], c2, nl[v]));
        if (MASK) p = (v >= lim) ? p : 0.f;
        const float ds = p * pacc[v];
        sacc[v] = p;
        pacc[v] = ds;
        amax = fmaxf(amax, fabsf(ds));
    }
    return amax;
}

// Adds a 32 x 64 dQ region, the accumulators acc0 / acc1 of two
// horizontally adjacent 32x32x64 MFMA tiles (lane = column, VGPR v = row
// 8 (v / 4) + 4 g + v % 4), into the FP16 accumulator so that every packed
// atomic instruction covers two whole 128-byte rows.  v_permlane32_swap
// first regroups the halves: its first result holds the lane-group-0 rows of
// both tiles (lanes 0-31 the left tile, 32-63 the right one), the second the
// group-1 rows, so lane l then holds column l of its rows.  Neighbour lanes
// then exchange halves so that each lane adds two adjacent columns of one
// row: the even lane of a pair takes the even row of each VGPR pair, the odd
// lane the odd one.  `region` is the region's first element, `rs` the row
// stride in elements; rows >= nrows are skipped.
template <bool CHECK>
__device__ __forceinline__ void dq_region_atomics(const v16f& acc0, const v16f& acc1,
                                                  _Float16* region, size_t rs, int lane, int nrows)
{
    const bool odd = lane & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
    const uint32_t lane_off = (uint32_t)((((size_t)(odd ? 1 : 0)) * rs + (lane & 62)) * 2);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int v = 2 * p;
            const auto lo = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0[v]),
                                                             __float_as_uint(acc1[v]), false, false);
            const auto hi = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0[v + 1]),
                                                             __float_as_uint(acc1[v + 1]), false,
                                                             false);
            const h2 mine = __builtin_convertvector(
                v2f{__uint_as_float(lo[half]), __uint_as_float(hi[half])}, h2);
            const uint32_t w = __builtin_bit_cast(uint32_t, mine);
            const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xB1, 0xF, 0xF, false);
            const uint32_t out = __builtin_amdgcn_perm(y, w, sel);
            // rows of VGPR pair (v, v + 1): 8 (p / 2) + 2 (p % 2) + 4 half + {0, 1}
            const int roff = 8 * (p / 2) + 2 * (p % 2) + 4 * half;
            if (!CHECK || roff + (odd ? 1 : 0) < nrows)
                __builtin_amdgcn_global_atomic_fadd_v2f16(
                    (h2*)((char*)(region + (size_t)roff * rs) + lane_off), __builtin_bit_cast(h2, out));
        }
    }
}

// Workgroup of 8 waves in two roles, pipelined by one query tile.  Score
// waves (0-3) own the keys 32 w .. + 31 of the 128-key tile: for tile j they
// compute S and dP (32 keys x 64 queries), P, dS, the two 32 x 32 dS block
// exponents, and write P^ and dS^ key-major to LDS.  Gradient waves (4-7)
// own the same keys and, for tile j - 1, contract those P^ / dS^ rows with
// the staged dO and Q codes into dV and dK (all of the head dim, in
// registers) and compute their share of the tile's dQ.  The two waves that
// share a SIMD thus interleave an exponential-heavy and an MFMA-heavy
// instruction stream, and one barrier per tile suffices: Q / dO tiles are
// triple-buffered (staging j + 1, scores j, gradients j - 1) and P^ / dS^
// double-buffered.
//
// Exact modes (per-token exponents; review section 4 and jaehun.me section
// 3.2): an exponent that varies along an MFMA's contraction axis cannot ride
// in its 32-wide block scale, so it is folded into the other operand, whose
// FP32 values are scaled by 2^(e(token) - block maximum) just before their
// E4M3 rounding: the dO exponent into P^ (dV), the Q exponent into dS^ (dK)
// and the K exponent into the dQ copy of dS^, which carries one exponent per
// (query row, 32-key block).  In the normal E4M3 range this equals shifting
// the rounded codes, i.e. the unfolded products.  MODE_FP4 recomputes S from
// the E2M1 score views through the FP16 MFMA, as the forward does.
template <int D, bool WITH_DQ, int MODE>
__global__ __launch_bounds__(512) void bwd_kernel(AttnArgs a)
{
    using CT = CodeTile<D>;         // token-major code tiles (swizzled rows at D = 128)
    constexpr int PITCH16 = 2 * D + 16;
    constexpr int SPITCH = 64 + 16; // P^ / dS^ tiles, key-major: [128 keys][64 queries]
    constexpr int NKS = D / 64;
    constexpr int NKH = D / 16;
    constexpr int NDT = D / 32;
    constexpr int CPR = D / 16;
    constexpr bool EXACT = MODE != MODE_BLOCK;
    constexpr bool FP4 = MODE == MODE_FP4;
    __shared__ __attribute__((aligned(16))) uint8_t s_kt[128 * CT::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[3][64 * CT::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_do[3][64 * CT::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_p[2][128 * SPITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_ds[2][128 * SPITCH];
    __shared__ int s_eq[3][64], s_edo[3][64], s_kq[3][64];
    __shared__ __attribute__((aligned(16))) float s_nlse[3][64];
    __shared__ __attribute__((aligned(16))) float s_delta[3][64];
    __shared__ int s_dsexp[2][2][4];   // [buffer][query half][key group]
    __shared__ int s_ekb[4];
    // exact modes: the dQ copy of dS^ and its per-row exponents, the Q / dO
    // block maxima and fold factors; FP4: the FP16 expansion of the Q view
    __shared__ __attribute__((aligned(16))) uint8_t s_dsr[EXACT ? 2 : 1][EXACT ? 128 * SPITCH : 16];
    __shared__ __attribute__((aligned(16))) int s_er[EXACT ? 2 : 1][4][EXACT ? 64 : 1];
    __shared__ int s_eqb[3][2], s_egb[3][2];
    __shared__ __attribute__((aligned(16))) float s_fq[EXACT ? 3 : 1][64];
    __shared__ __attribute__((aligned(16))) float s_fg[EXACT ? 3 : 1][64];
    __shared__ __attribute__((aligned(16))) uint8_t s_q16[FP4 ? 2 : 1][FP4 ? 64 * PITCH16 : 16];

    const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
    const size_t T = (size_t)a.T;
    // Persistent: one workgroup per CU slot takes (item, kv head) tickets in
    // cost order from an atomic counter (zeroed with the work list), the
    // next ticket fetched while the current one runs, so no workgroup
    // dispatch and no ticket latency sits between items.
    __shared__ int s_ticket[2];
    int* const next_ticket = a.tickets;
    const int ntickets = *a.count * Hkv;
    if (threadIdx.x == 0) s_ticket[0] = atomicAdd(next_ticket, 1);
    __syncthreads();
    for (int slot = 0;; slot ^= 1) {
        const int ticket = __builtin_amdgcn_readfirstlane(s_ticket[slot]);
        if (ticket >= ntickets) break;  // uniform: every thread read the slot after a barrier
        // the thread index is re-read per item (opaque to the compiler), so
        // lane-dependent offsets are recomputed per item instead of being
        // held in registers across the whole loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = wave_id(), g = lane >> 5;
        const int kg = wave & 3;
        const bool scorer = wave < 4;
        if (tid == 0) s_ticket[slot ^ 1] = atomicAdd(next_ticket, 1);
        const int item = ticket / Hkv, hk = ticket % Hkv;
        const int b = a.items[2 * item], kt = a.items[2 * item + 1];
        const int s = a.cu[b], e = a.cu[b + 1];
        const int k0 = s + 128 * kt;
        const int kw0 = k0 + 32 * kg;
        const int kj = kw0 + (lane & 31);
        const bool kvalid = kj < e;
        const bool wave_keys = kw0 < e;
        const float c2 = a.c2;
        const int krow = 32 * kg + (lane & 31);  // this lane's key in the key-major tiles

        // the workgroup's K tile, token-major, for the dQ MFMA (k = keys)
        for (int c = tid; c < 128 * CPR; c += 512) {
            const int row = c / CPR, col = 16 * (c % CPR);
            const int t = k0 + row;
            v4i kv = {0, 0, 0, 0};
            if (t < e) kv = *(const v4i*)(a.k_codes + ((size_t)t * Hkv + hk) * D + col);
            *(v4i*)(s_kt + CT::off(row, col)) = kv;
        }
        // K block exponents of the dQ MFMA (lane = key of block kg); with
        // per-token exponents the block maximum and this key's fold factor
        const int ek = kvalid ? (int)a.k_exps[(size_t)hk * T + kj] : 127;
        float fk = 1.f;
        if constexpr (EXACT) {
            const uint32_t ekb = half_wave_max_u32(kvalid ? (uint32_t)ek : 0u);
            fk = kvalid ? ldexpf(1.f, ek - (int)ekb) : 0.f;
            if (scorer && lane == 0) s_ekb[kg] = (int)ekb;
        } else {
            if (tid < 4)
                s_ekb[tid] = (k0 + 32 * tid < e) ? (int)a.k_exps[(size_t)hk * T + k0 + 32 * tid] : 127;
        }

        // iterations: q heads of the group (outer) x 64-query tiles that see the keys
        const int qt_lo = a.causal ? 2 * kt : 0;
        const int nqt = (e - s + 63) / 64 - qt_lo;
        const int niter = G * nqt;
        auto tile_head = [&](int j) { return hk * G + j / nqt; };
        auto tile_base = [&](int j) { return s + 64 * (qt_lo + j % nqt); };

        // The score waves (threads 0-255) fetch and stage the query tiles, so
        // the gradient waves' dQ atomics never sit ahead of a load they must wait
        // for.  Every staging thread writes (the waves write identical
        // statistics), so that every prefetched register is consumed on every
        // path.
        using Tile = QTile<D, 256>;
        auto stage = [&](const Tile& r, int buf, int buf2) {
#pragma unroll
            for (int k = 0; k < Tile::NC; ++k) {
                const int c = tid + 256 * k;
                const bool isq = c < 4 * D;
                const int cc = isq ? c : c - 4 * D;
                const int row = cc / CPR, col = 16 * (cc % CPR);
                *(v4i*)((isq ? s_q[buf] : s_do[buf]) + CT::off(row, col)) = r.c[k];
            }
            const int row = tid & 63;
            s_eq[buf][row] = r.ok ? r.eq : 127;
            s_edo[buf][row] = r.ok ? r.edo : 127;
            s_kq[buf][row] = r.ok ? r.pre + a.scale_exp : 0;
            // 8 - LSE log2 e: exp2 of the score term then yields 256 P; rows past
            // the document end get -inf, so their P is exactly zero
            s_nlse[buf][row] = r.ok ? boosted_row_term(r.lse) : -INFINITY;
            s_delta[buf][row] = r.ok ? r.delta : 0.f;
            if constexpr (EXACT) {
                // lane = query row: block maxima of the Q and dO exponents over
                // each 32-query half and the rows' fold factors
                const uint32_t eqr = r.ok ? (uint32_t)r.eq : 0u, egr = r.ok ? (uint32_t)r.edo : 0u;
                const uint32_t eqb = half_wave_max_u32(eqr), egb = half_wave_max_u32(egr);
                s_eqb[buf][row >> 5] = (int)eqb;
                s_egb[buf][row >> 5] = (int)egb;
                s_fq[buf][row] = r.ok ? ldexpf(1.f, (int)eqr - (int)eqb) : 0.f;
                s_fg[buf][row] = r.ok ? ldexpf(1.f, (int)egr - (int)egb) : 0.f;
            }
            if constexpr (FP4) {
                // the Q row's features (tid % 4) D / 4 .. + D / 4 - 1 as FP16
                uint8_t* dst = &s_q16[buf2][(tid >> 2) * PITCH16 + 2 * (tid & 3) * (D / 4)];
#pragma unroll
                for (int q = 0; q < D / 32; ++q) {
                    const float sc = __builtin_amdgcn_cvt_f32_fp8((int)((r.q4s >> (8 * (q / 2))) & 0xff), 0);
                    *(h8*)(dst + 16 * q) = fp4x8_to_f16((uint32_t)r.q4[q], sc);
                }
            }
        };
        Tile nxt;
        auto prefetch = [&](int j) {
            const int j1 = min(j + 1, niter - 1);
            load_qtile<D, 256, MODE>(a, nxt, tile_head(j1), tile_base(j1), e, tid);
        };

        if (scorer) {
            load_qtile<D, 256, MODE>(a, nxt, tile_head(0), tile_base(0), e, tid);
            stage(nxt, 0, 0);
        }
        // every load issued so far has landed (vmcnt(0)), so that inside the loop
        // only the prefetch of the next tile is outstanding
        __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();

        if (scorer) {
            // this wave's K and V rows: B operands of S = Q K^T (E4M3 codes, or
            // the FP16 expansion of the E2M1 view) and dP = dO V^T
            v8i kf[FP4 ? 1 : NKS], vf[NKS];
            h8 kh[FP4 ? NKH : 1];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if (kvalid) {
                    if constexpr (!FP4)
                        kf[ks] = row_operand(a.k_codes + ((size_t)kj * Hkv + hk) * D + 64 * ks, lane);
                    vf[ks] = row_operand(a.v_codes + ((size_t)kj * Hkv + hk) * D + 64 * ks, lane);
                } else {
                    if constexpr (!FP4) kf[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                    vf[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
                }
            }
            if constexpr (FP4) {
                const size_t row = (size_t)min(kj, e - 1) * Hkv + hk;
#pragma unroll
                for (int ks = 0; ks < NKH; ++ks) {
                    const uint32_t c = *(const uint32_t*)(a.k_fp4 + row * (D / 2) + 8 * ks + 4 * g);
                    const float sc = __builtin_amdgcn_cvt_f32_fp8((int)a.k_fp4_scales[row * (D / 16) + ks], 0);
                    kh[ks] = fp4x8_to_f16(c, sc);
                }
            }
            const int ev = kvalid ? (int)a.v_exps[(size_t)hk * T + kj] : 127;
            __builtin_amdgcn_s_waitcnt(0x0F70);

            for (int j = 0; j <= niter; ++j) {
                prefetch(j);
                if (j < niter) {
                    const int c3 = j % 3, pb = j & 1;
                    const int qb = tile_base(j);
                    const uint8_t* sq = s_q[c3];
                    const uint8_t* sg = s_do[c3];
                    // the two 32 x 32 blocks (queries 32 t .. + 31 of the tile):
                    // all S / dP MFMAs first, then the element-wise work
                    bool active[2];
                    v16f sacc[2], pacc[2];
                    // the rows' statistics (8 - LSE log2 e and D) into registers
                    // ahead of the MFMAs, so their LDS latency overlaps them (not
                    // with the FP16 score path, whose registers are spoken for)
                    float nlv[2][16], dlv[2][16];
#pragma unroll
                    for (int t = 0; t < (FP4 ? 0 : 2); ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float4 x = *(const float4*)&s_nlse[c3][32 * t + 16 * g + 4 * i];
                            const float4 y = *(const float4*)&s_delta[c3][32 * t + 16 * g + 4 * i];
#pragma unroll
                            for (int k = 0; k < 4; ++k) {
                                nlv[t][4 * i + k] = k == 0 ? x.x : k == 1 ? x.y : k == 2 ? x.z : x.w;
                                dlv[t][4 * i + k] = k == 0 ? y.x : k == 1 ? y.y : k == 2 ? y.z : y.w;
                            }
                        }
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        active[t] = wave_keys && (!a.causal || qb + 32 * t + 31 >= kw0);
#pragma unroll
                        for (int v = 0; v < 16; ++v) sacc[t][v] = pacc[t][v] = 0.f;
                        if (active[t]) {
                            const int qr = perm_row(t, lane & 31);
                            const int edr = s_edo[c3][qr];
                            if constexpr (FP4) {
#pragma unroll
                                for (int ks = 0; ks < NKH; ++ks)
                                    sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                        *(const h8*)(s_q16[pb] + qr * PITCH16 + 2 * (16 * ks + 8 * g)), kh[ks],
                                        sacc[t], 0, 0, 0);
                            } else {
                                const int eqr = s_eq[c3][qr];
#pragma unroll
                                for (int ks = 0; ks < NKS; ++ks)
                                    sacc[t] = mfma_f8(tile_row_operand<D>(sq, qr, 64 * ks, lane), kf[ks],
                                                      sacc[t], eqr, ek);
                            }
#pragma unroll
                            for (int ks = 0; ks < NKS; ++ks)
                                pacc[t] = mfma_f8(tile_row_operand<D>(sg, qr, 64 * ks, lane), vf[ks],
                                                  pacc[t], edr, ev);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        v4i pf = {0, 0, 0, 0}, df = {0, 0, 0, 0}, dfr = {0, 0, 0, 0};
                        int dse = 127;
                        int er[16];
#pragma unroll
                        for (int v = 0; v < 16; ++v) er[v] = 0;
                        if (active[t]) {
                            // Masking is needed only where some key is invalid or,
                            // causally, some query precedes some key; queries past
                            // the document end have 256 P = exp2(-inf) = 0 and
                            // D = 0.  Element v of lane group g is query
                            // qb + 32 t + 16 g + v.
                            const int q0 = 32 * t + 16 * g;
                            const float* nl = FP4 ? &s_nlse[c3][q0] : nlv[t];
                            const float* dl = FP4 ? &s_delta[c3][q0] : dlv[t];
                            const bool full = kw0 + 32 <= e && (!a.causal || qb + 32 * t >= kw0 + 31);
                            float amax;
                            if (full) {
                                amax = softmax_grad<false>(sacc[t], pacc[t], nl, dl, c2, 0);
                            } else {
                                const int lim = a.causal ? kj - qb - 32 * t - 16 * g : (kvalid ? -1 : 16);
                                amax = softmax_grad<true>(sacc[t], pacc[t], nl, dl, c2, lim);
                            }
                            // block exponent of dS = 2^-8 (256 dS); the scaling is exact
                            const int et = ceil_exp448(wave_max_nonneg(amax) * 0.00390625f);
                            dse = et + 127;
                            if constexpr (EXACT) {
                                // per-row exponents of the dQ copy: each query
                                // row's largest |dS| over this block's 32 keys,
                                // one row per lane, then all 16 rows of the lane
                                // group back from LDS (the same wave's write)
                                uint32_t ab[16];
#pragma unroll
                                for (int v = 0; v < 16; ++v) ab[v] = __float_as_uint(fabsf(pacc[t][v]));
                                const int erl = ceil_exp448(
                                    __uint_as_float(row_max_transpose(ab, lane)) * 0.00390625f);
                                int* erow = &s_er[pb][kg][32 * t + 16 * g];
                                if ((lane & 16) == 0) erow[rev4(lane & 15)] = erl + 127;
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const v4i e4 = *(const v4i*)(erow + 4 * q);
                                    er[4 * q] = e4.x - 127;
                                    er[4 * q + 1] = e4.y - 127;
                                    er[4 * q + 2] = e4.z - 127;
                                    er[4 * q + 3] = e4.w - 127;
                                }
                                const float* fg = &s_fg[c3][q0];
                                const float* fq = &s_fq[c3][q0];
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    float pv[4], dv4[4], rv[4];
#pragma unroll
                                    for (int k = 0; k < 4; ++k) {
                                        const int v = 4 * q + k;
                                        pv[k] = sacc[t][v] * fg[v];
                                        dv4[k] = ldexpf(pacc[t][v] * fq[v], -et - 8);
                                        rv[k] = ldexpf(pacc[t][v] * fk, -er[v] - 8);
                                    }
                                    pf[q] = (int)cvt4_fp8(pv[0], pv[1], pv[2], pv[3]);
                                    df[q] = (int)cvt4_fp8(dv4[0], dv4[1], dv4[2], dv4[3]);
                                    dfr[q] = (int)cvt4_fp8(rv[0], rv[1], rv[2], rv[3]);
                                }
                            } else {
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    pf[q] = (int)cvt4_fp8(sacc[t][4 * q], sacc[t][4 * q + 1],
                                                          sacc[t][4 * q + 2], sacc[t][4 * q + 3]);
                                    df[q] = (int)cvt4_fp8_div(pacc[t][4 * q], pacc[t][4 * q + 1],
                                                              pacc[t][4 * q + 2], pacc[t][4 * q + 3],
                                                              ds_code_divisor(et));
                                }
                            }
                        }
                        // key-major rows: 16 bytes at the block's queries and lane group
                        *(v4i*)(s_p[pb] + krow * SPITCH + 32 * t + 16 * g) = pf;
                        *(v4i*)(s_ds[pb] + krow * SPITCH + 32 * t + 16 * g) = df;
                        if (lane == 0) s_dsexp[pb][t][kg] = dse;
                        if constexpr (EXACT) {
                            *(v4i*)(s_dsr[pb] + krow * SPITCH + 32 * t + 16 * g) = dfr;
                            if (!active[t] && (lane & 16) == 0) s_er[pb][kg][32 * t + 16 * g + (lane & 15)] = 127;
                        }
                    }
                }
                stage(nxt, (j + 1) % 3, (j + 1) & 1);
                lds_barrier();
            }
        } else {
            // dK^T, dV^T of the wave's keys over the whole head dim
            v16f dk[NDT], dv[NDT];
#pragma unroll
            for (int i = 0; i < NDT; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) dk[i][v] = dv[i][v] = 0.f;
            const size_t dq_rs = (size_t)Hq * D;  // row stride of the dQ accumulator

            for (int j = 0; j <= niter; ++j) {
                if (j >= 1) {
                    const int jp = j - 1;
                    const int c3 = jp % 3, pb = jp & 1;
                    const int qb = tile_base(jp), h = tile_head(jp);
                    const uint8_t* sq = s_q[c3];
                    const uint8_t* sg = s_do[c3];
                    // dV^T += dO^T P^ and dK^T += Q^T dS^ over the tile's 64
                    // queries (k); the B operands are the key's P^ / dS^ rows in
                    // the k layout (bytes 0-15 query half 0, 16-31 half 1)
                    if (wave_keys && (!a.causal || qb + 63 >= kw0)) {
                        const v4i p0 = *(const v4i*)(s_p[pb] + krow * SPITCH + 16 * g);
                        const v4i p1 = *(const v4i*)(s_p[pb] + krow * SPITCH + 32 + 16 * g);
                        const v4i d0 = *(const v4i*)(s_ds[pb] + krow * SPITCH + 16 * g);
                        const v4i d1 = *(const v4i*)(s_ds[pb] + krow * SPITCH + 32 + 16 * g);
                        const v8i pfull = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                        const v8i dfull = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
                        const int sdo = EXACT ? s_egb[c3][g] : s_edo[c3][32 * g];
                        const int sqe = EXACT ? s_eqb[c3][g] : s_eq[c3][32 * g];
                        const int dsg = s_dsexp[pb][g][kg];
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) {
                            dv[dt] = mfma_f8(tile_tr_operand<D>(sg, 0, 32 * dt, lane), pfull, dv[dt],
                                             sdo, kScaleMinus8);
                            dk[dt] = mfma_f8(tile_tr_operand<D>(sq, 0, 32 * dt, lane), dfull, dk[dt],
                                             sqe, dsg);
                        }
                    }

                    if constexpr (WITH_DQ) {
                        // dQ = dS^ K^ over the tile's 128 keys: wave kg computes the
                        // 32 x 64 region (query half ct, head-dim tiles dt0, dt0 + 1).
                        // The row's prescale 2^(k_i + f) (2^f <= softmax scale <
                        // 2^(f + 1)) rides in the A operand's block scale; the
                        // finalize applies the remaining scale 2^-(k_i + f).
                        if (kg < NDT) {
                            const int ct = kg / (NDT / 2), dt0 = 2 * (kg % (NDT / 2));
                            const int nrows = e - (qb + 32 * ct);
                            if (nrows > 0) {
                                const int qrow = 32 * ct + (lane & 31);
                                const int kq = s_kq[c3][qrow];
                                const int e0 = EXACT ? s_er[pb][g][qrow] : s_dsexp[pb][ct][g];
                                const int e1 = EXACT ? s_er[pb][2 + g][qrow] : s_dsexp[pb][ct][2 + g];
                                const int sa0 = min(max(e0 + kq, 0), 254);
                                const int sa1 = min(max(e1 + kq, 0), 254);
                                const uint8_t* sdq = EXACT ? s_dsr[pb] : s_ds[pb];
                                const v8i a0 = lds_tr_operand(sdq, SPITCH, 0, 32 * ct, lane);
                                v16f acc[2];
#pragma unroll
                                for (int i = 0; i < 2; ++i) {
#pragma unroll
                                    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
                                    acc[i] = mfma_f8(a0, tile_tr_operand<D>(s_kt, 0, 32 * (dt0 + i), lane),
                                                     acc[i], sa0, s_ekb[g]);
                                }
                                if (k0 + 64 < e) {
                                    const v8i a1 = lds_tr_operand(sdq + 64 * SPITCH, SPITCH, 0, 32 * ct, lane);
#pragma unroll
                                    for (int i = 0; i < 2; ++i)
                                        acc[i] = mfma_f8(a1, tile_tr_operand<D>(s_kt, 64,
                                                                            32 * (dt0 + i), lane),
                                                         acc[i], sa1, s_ekb[2 + g]);
                                }
                                _Float16* region = a.dq_acc + ((size_t)(qb + 32 * ct) * Hq + h) * D + 32 * dt0;
                                if (nrows >= 32)
                                    dq_region_atomics<false>(acc[0], acc[1], region, dq_rs, lane, nrows);
                                else
                                    dq_region_atomics<true>(acc[0], acc[1], region, dq_rs, lane, nrows);
                            }
                        }
                    }
                }
                lds_barrier();
            }

            // rotated Q and K: dK = dK_r H (the Sylvester matrix, unnormalised;
            // the softmax scale already carries the 1 / d)
            if (a.rotate) fwht_cols<NDT>(dk, lane);
            if (kvalid) {
                uint16_t* krp = a.dk + ((size_t)kj * Hkv + hk) * D;
                uint16_t* vrp = a.dv + ((size_t)kj * Hkv + hk) * D;
                const float sc = a.scale;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        v2i wk, wv;
                        wk.x = (int)pack_bf16x2(dk[dt][4 * q] * sc, dk[dt][4 * q + 1] * sc);
                        wk.y = (int)pack_bf16x2(dk[dt][4 * q + 2] * sc, dk[dt][4 * q + 3] * sc);
                        wv.x = (int)pack_bf16x2(dv[dt][4 * q], dv[dt][4 * q + 1]);
                        wv.y = (int)pack_bf16x2(dv[dt][4 * q + 2], dv[dt][4 * q + 3]);
                        *(v2i*)(krp + 32 * dt + 8 * q + 4 * g) = wk;
                        *(v2i*)(vrp + 32 * dt + 8 * q + 4 * g) = wv;
                    }
            }
        }
        // item boundary: every wave is done with this item's LDS before the next
        // item's first writes, and the next ticket is visible
        __syncthreads();
    }  // tickets
}

// Adds one 32 x 32 dQ tile, the accumulator of a 32x32x64 MFMA (lane =
// column, VGPR v = row 8 (v / 4) + 4 g + v % 4), into the FP16 accumulator
// with packed atomics of two adjacent columns: VGPRs v, v + 1 (rows r, r + 1
// of the lane's column c) are converted as one FP16 pair, neighbour lanes
// swap pairs (DPP) and v_perm regroups them, so that the even lane of a pair
// adds (row r; columns c, c + 1) and the odd lane (row r + 1; columns c - 1,
// c).  The atomics are buffer atomics on a resource based at the tile's first
// row: each row pair's byte offset is a scalar (soffset), the lane's a
// constant VGPR, so no atomic needs 64-bit vector address arithmetic.  Rows
// >= nrows are skipped.
template <bool CHECK>
__device__ __forceinline__ void dq_tile_atomics_pk(const v16f& acc, _Float16* tile, uint32_t rs_bytes, int lane,
                                                   int nrows)
{
    // recomputed per call: the row offsets are a few scalar multiplies, not
    // eight values held across the loop
    asm volatile("" : "+s"(rs_bytes));
    const bool odd = lane & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
    const int lrow = 4 * (lane >> 5) + (odd ? 1 : 0);
    const uint32_t lane_off = (uint32_t)lrow * rs_bytes + 2 * (uint32_t)(lane & 30);
    // raw buffer (stride 0), no range limit; data format word of gfx9
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(tile, 0, -1, 0x00020000);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int v = 2 * p;
        const int r0 = 8 * (v / 4) + (v % 4);
        const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{acc[v], acc[v + 1]}, h2));
        const uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xB1, 0xF, 0xF, false);
        const uint32_t out = __builtin_amdgcn_perm(y, w, sel);
        // (readfirstlane: the offset stays a scalar where the row checks
        // make the control flow merge)
        const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)r0 * rs_bytes);
        if (!CHECK || r0 + lrow < nrows)
            (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_v2f16(__builtin_bit_cast(h2, out), rsrc, lane_off, soff,
                                                                    0);
    }
}

// The per-query statistics of one 64-query tile (lane = query, rows past the
// document end clamped to its last row and marked invalid).
struct QStats {
    int eq, edo, pre, ok;
    float lse, delta;
};

__device__ __forceinline__ void load_qstats(const AttnArgs& a, QStats& r, int h, int qb, int e, int tid)
{
    const int t = qb + (tid & 63);
    r.ok = t < e;
    const size_t i = (size_t)h * a.T + min(t, e - 1);
    r.eq = a.q_exps[i];
    r.edo = a.do_exps[i];
    r.lse = a.lse_in[i];
    r.delta = a.delta[i];
    r.pre = a.prescale[i];
}

// Writes one wave's dK and dV rows (lane = key kj, accumulators of the
// 32 x 32 MFMA layout over the head dim) as bf16: dK times the softmax scale,
// and, with rotated Q and K, dK = dK_r H (the Sylvester matrix,
// unnormalised; the scale already carries the 1 / d).  Keys past the
// document end are not written.
template <int D>
__device__ __forceinline__ void store_dkdv(const AttnArgs& a, v16f (&dk)[D / 32], v16f (&dv)[D / 32], int kj,
                                           int e, int hk, int lane)
{
    constexpr int NDT = D / 32;
    const int g = lane >> 5;
    if (a.rotate) fwht_cols<NDT>(dk, lane);
    if (kj >= e) return;
    uint16_t* krp = a.dk + ((size_t)kj * a.Hkv + hk) * D;
    uint16_t* vrp = a.dv + ((size_t)kj * a.Hkv + hk) * D;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v2i wk, wv;
            wk.x = (int)pack_bf16x2(dk[dt][4 * q] * sc, dk[dt][4 * q + 1] * sc);
            wk.y = (int)pack_bf16x2(dk[dt][4 * q + 2] * sc, dk[dt][4 * q + 3] * sc);
            wv.x = (int)pack_bf16x2(dv[dt][4 * q], dv[dt][4 * q + 1]);
            wv.y = (int)pack_bf16x2(dv[dt][4 * q + 2], dv[dt][4 * q + 3]);
            *(v2i*)(krp + 32 * dt + 8 * q + 4 * g) = wk;
            *(v2i*)(vrp + 32 * dt + 8 * q + 4 * g) = wv;
        }
}

// Backward over document-local 256-key tiles (token-block operands).  A
// workgroup of 8 waves owns 256 keys of one kv head; wave w owns keys
// 32 w .. 32 w + 31 in every role: for each 64-query tile it forms S and dP
// for them (one 32-query half at a time), P, dS and their codes, and
// contracts those codes with the tile's dO and Q into its keys' dV and dK,
// accumulated over the head dim in registers across the whole loop (the GQA
// head reduction without atomics).  dS^ also goes key-major to LDS, where the
// tile's dQ = dS^ K^ over all 256 keys is formed one step later, one FP16
// partial per query row and 256-key tile (half the atomic payload of 128-key
// tiles).
//
// Each step every wave first forms and adds (packed FP16 atomics) its 32 x 32
// tile of the dQ of query tile j - 1 (D = 64: waves 4-7 only), then forms
// the scores of tile j for its keys and contracts them.  Waves 0-3 also
// fetch the next Q / dO tile (at D = 128 straight into LDS,
// global_load_lds), issued before their atomics: vector memory counters
// complete in order, and the wait for the fetch at the end of the step then
// also covers atomics issued a whole step earlier.  Q / dO tiles are
// double-buffered (tile j in use, j + 1 landing), dS^ double-buffered; one
// barrier per step orders the LDS traffic.
template <int D, bool WITH_DQ, int MODE>
__global__ __launch_bounds__(512) void bwd_wide_kernel(AttnArgs a)
{
    using CT = CodeTile<D>;
    constexpr int NKEY = 256;
    constexpr int SPITCH = 64 + 16;  // dS^ tile, key-major: [256 keys][64 queries]
    constexpr int PITCH16 = 2 * D + 16;
    constexpr int NKS = D / 64;
    constexpr int NKH = D / 16;
    constexpr int NDT = D / 32;
    constexpr int CPR = D / 16;
    constexpr bool DMA = CT::SWZ;    // D = 128: Q / dO tiles by direct global -> LDS loads
    constexpr bool EXACT = MODE != MODE_BLOCK;
    constexpr bool FP4 = MODE == MODE_FP4;
    static_assert(!EXACT || D == 64, "per-token operands: 256-key tiles at d = 64 only");
    // code tiles 128-byte aligned (swz_row_operand addresses them by XOR)
    __shared__ __attribute__((aligned(128))) uint8_t s_kt[NKEY * CT::PITCH];
    __shared__ __attribute__((aligned(128))) uint8_t s_vt[NKEY * CT::PITCH];
    __shared__ __attribute__((aligned(128))) uint8_t s_q[2][64 * CT::PITCH];
    __shared__ __attribute__((aligned(128))) uint8_t s_do[2][64 * CT::PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_ds[2][NKEY * SPITCH];
    __shared__ int s_eq[2][64], s_edo[2][64];
    // the rows' prescale exponents are read by the dQ of tile j - 1 while tile
    // j + 1's are staged: three slots (tile % 3)
    __shared__ int s_kq[3][64];
    __shared__ __attribute__((aligned(16))) float s_nlse[2][64];
    __shared__ __attribute__((aligned(16))) float s_ndelta[2][64];  // -D
    __shared__ int s_dsexp[2][2][8];  // [buffer][query half][key block]
    __shared__ int s_ekb[8];
    __shared__ int s_ticket[2];
    // per-token operands: the dQ copy's per-(row, key block) exponents and
    // their code multipliers 2^(-e - 8), the Q / dO exponent maxima per
    // 32-query half and the rows' Q fold factors; E2M1 score view: the FP16
    // expansion of the Q view
    __shared__ __attribute__((aligned(16))) int s_er[EXACT ? 2 : 1][8][EXACT ? 64 : 1];
    __shared__ __attribute__((aligned(16))) float s_rm[EXACT ? 2 : 1][8][EXACT ? 64 : 1];
    __shared__ int s_eqb[2][2], s_egb[2][2];
    __shared__ __attribute__((aligned(16))) float s_fq[EXACT ? 2 : 1][64];
    __shared__ __attribute__((aligned(16))) uint8_t s_q16[FP4 ? 2 : 1][FP4 ? 64 * PITCH16 : 16];

    const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
    const size_t T = (size_t)a.T;
    int* const next_ticket = a.tickets;
    // the count[2] costliest items are split into two tickets per kv head
    // (tickets 2 p, 2 p + 1 for pair p = item x Hkv + kv head), the rest take
    // one ticket per kv head
    const int npairs = a.count[2] * Hkv;
    const int ntickets = *a.count * Hkv + npairs;
    if (threadIdx.x == 0) s_ticket[0] = atomicAdd(next_ticket, 1);
    __syncthreads();
    for (int slot = 0;; slot ^= 1) {
        const int ticket = __builtin_amdgcn_readfirstlane(s_ticket[slot]);
        if (ticket >= ntickets) break;  // uniform: every thread read the slot after a barrier
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = wave_id(), g = lane >> 5;
        if (tid == 0) s_ticket[slot ^ 1] = atomicAdd(next_ticket, 1);
        const int pair = ticket < 2 * npairs ? ticket >> 1 : ticket - npairs;
        const int half = ticket < 2 * npairs ? (ticket & 1) : -1;  // -1: whole item
        const int item = pair / Hkv, hk = pair % Hkv;
        const int b = a.items[2 * item], kt = a.items[2 * item + 1];
        const int s = a.cu[b], e = a.cu[b + 1];
        const int k0 = s + NKEY * kt;
        const int kw0 = k0 + 32 * wave;
        const int kj = kw0 + (lane & 31);
        const bool kvalid = kj < e;
        const bool wave_keys = kw0 < e;
        const float c2 = a.c2;

        // the item's K and V tiles, token-major.  D = 128 and every key inside
        // the document: direct loads into the swizzled tiles (wave w fills
        // rows 32 w .. + 31 with four loads of eight rows each), landing by the
        // asm wait before the loop together with the first Q / dO tile, so the
        // item start waits for one memory round trip, not two
        if (DMA && k0 + NKEY <= e) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rb = 32 * wave + 8 * i;
                const int row = rb + (lane >> 3);
                const size_t src = ((size_t)(k0 + row) * Hkv + hk) * D + 16 * ((lane & 7) ^ tile_swizzle(row));
                dma16_opaque(a.k_codes + src, (lds_void*)&s_kt[rb * 128]);
                dma16_opaque(a.v_codes + src, (lds_void*)&s_vt[rb * 128]);
            }
        } else
        for (int c = tid; c < NKEY * CPR; c += 512) {
            const int row = c / CPR, col = 16 * (c % CPR);
            const int t = k0 + row;
            v4i kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (t < e) {
                kv = *(const v4i*)(a.k_codes + ((size_t)t * Hkv + hk) * D + col);
                vv = *(const v4i*)(a.v_codes + ((size_t)t * Hkv + hk) * D + col);
            }
            *(v4i*)(s_kt + CT::off(row, col)) = kv;
            *(v4i*)(s_vt + CT::off(row, col)) = vv;
        }
        const int ek = kvalid ? (int)a.k_exps[(size_t)hk * T + kj] : 127;
        const int ev = kvalid ? (int)a.v_exps[(size_t)hk * T + kj] : 127;
        // K block exponents of the dQ MFMA; with per-token exponents the
        // maximum over the wave's 32 keys, and this key's fold factor
        // 2^(e_K - max) as the divisor 2^(max - e_K) of the scaled conversion
        // (capped at 2^127, where every code is zero anyway; 1 past the
        // document end, where dS is zero)
        float fkdiv = 1.f;
        if constexpr (EXACT) {
            const uint32_t ekb = half_wave_max_u32(kvalid ? (uint32_t)ek : 0u);
            fkdiv = kvalid ? ldexpf(1.f, min((int)ekb - ek, 127)) : 1.f;
            if (lane == 0) s_ekb[wave] = (int)ekb;
        } else {
            if (tid < 8)
                s_ekb[tid] = (k0 + 32 * tid < e) ? (int)a.k_exps[(size_t)hk * T + k0 + 32 * tid] : 127;
        }
        // E2M1 score view: this lane's key row, expanded to FP16 (B operand of S)
        h8 kh[FP4 ? NKH : 1];
        if constexpr (FP4) {
            const size_t row = (size_t)min(kj, e - 1) * Hkv + hk;
#pragma unroll
            for (int ks = 0; ks < NKH; ++ks) {
                const uint32_t c = *(const uint32_t*)(a.k_fp4 + row * (D / 2) + 8 * ks + 4 * g);
                const float sc = __builtin_amdgcn_cvt_f32_fp8((int)a.k_fp4_scales[row * (D / 16) + ks], 0);
                kh[ks] = fp4x8_to_f16(c, sc);
            }
        }

        // iterations: q heads of the group (outer) x 64-query tiles that see the keys
        const int qt_lo = a.causal ? (NKEY / 64) * kt : 0;
        const int nqt = (e - s + 63) / 64 - qt_lo;
        // a split item's halves take iterations [0, n / 2) and [n / 2, n)
        const int nall = G * nqt;
        const int jlo = half == 1 ? nall / 2 : 0;
        const int niter = half == 0 ? nall / 2 : nall;
        auto tile_head = [&](int j) { return hk * G + j / nqt; };
        auto tile_base = [&](int j) { return s + 64 * (qt_lo + j % nqt); };

        // Q / dO tile j into buffer j & 1 (threads 0-255).  D = 128: wave w
        // fills rows 16 w .. + 15 of each tile with two direct loads of 1 KB
        // (eight rows), lane L writing LDS bytes 16 L .. + 15 of its block:
        // row + L / 8, physical chunk L % 8, i.e. logical chunk (L % 8) ^
        // tile_swizzle(row).  The loads are inline assembly: with the builtin
        // the compiler waits for them (vmcnt(0)) before the first LDS read of
        // the dQ product that follows, which only reads other tiles; the step
        // ends with an asm wait instead.  D = 64: through registers.
        using Tile = QTile<D, 256>;
        Tile nxt;
        QStats st;
        auto fetch = [&](int j) {
            const int h = tile_head(j), qb = tile_base(j);
            if constexpr (DMA) {
                const int buf = j & 1;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int rb = 16 * wave + 8 * i;
                    const int row = rb + (lane >> 3);
                    const int c = (lane & 7) ^ tile_swizzle(row);
                    const size_t src = ((size_t)min(qb + row, e - 1) * Hq + h) * D + 16 * c;
                    dma16_opaque(a.q_codes + src, (lds_void*)&s_q[buf][rb * 128]);
                    dma16_opaque(a.do_codes + src, (lds_void*)&s_do[buf][rb * 128]);
                }
                load_qstats(a, st, h, qb, e, tid);
            } else {
                load_qtile<D, 256, MODE>(a, nxt, h, qb, e, tid);
            }
        };
        auto stage = [&](int j) {
            const int buf = j & 1;
            int eq, edo, pre, ok;
            float lse, delta;
            if constexpr (DMA) {
                eq = st.eq; edo = st.edo; pre = st.pre; ok = st.ok; lse = st.lse; delta = st.delta;
            } else {
#pragma unroll
                for (int k = 0; k < Tile::NC; ++k) {
                    const int c = tid + 256 * k;
                    const bool isq = c < 4 * D;
                    const int cc = isq ? c : c - 4 * D;
                    const int row = cc / CPR, col = 16 * (cc % CPR);
                    *(v4i*)((isq ? s_q[buf] : s_do[buf]) + CT::off(row, col)) = nxt.c[k];
                }
                eq = nxt.eq; edo = nxt.edo; pre = nxt.pre; ok = nxt.ok; lse = nxt.lse; delta = nxt.delta;
            }
            const int row = tid & 63;
            s_eq[buf][row] = ok ? eq : 127;
            s_kq[j % 3][row] = ok ? pre + a.scale_exp : 0;
            if constexpr (EXACT) {
                // lane = query row: the Q and dO exponent maxima over each
                // 32-query half (the dK / dV MFMA scales) and the rows' Q fold
                // factors.  The dO fold 2^(e_dO - max) of P^ enters through the
                // exponent term, 2^(8 + e_dO - max - LSE log2 e), which makes
                // P 2^(e_dO - max) times larger; dP - D is made as much smaller
                // by taking the half's maximum as the dO rows' scale of the dP
                // product and D scaled to match, so dS itself is unchanged.
                const uint32_t eqr = ok ? (uint32_t)eq : 0u, egr = ok ? (uint32_t)edo : 0u;
                const uint32_t eqb = half_wave_max_u32(eqr), egb = half_wave_max_u32(egr);
                const int lfg = (int)egr - (int)egb;
                s_eqb[buf][row >> 5] = (int)eqb;
                s_egb[buf][row >> 5] = (int)egb;
                s_edo[buf][row] = (int)egb;
                s_fq[buf][row] = ok ? ldexpf(1.f, (int)eqr - (int)eqb) : 0.f;
                s_nlse[buf][row] = ok ? boosted_row_term(lse, lfg) : -INFINITY;
                s_ndelta[buf][row] = ok ? ldexpf(-delta, -lfg) : 0.f;
            } else {
                s_edo[buf][row] = ok ? edo : 127;
                // 8 - LSE log2 e: exp2 of the score term then yields 256 P; rows
                // past the document end get -inf, so their P is exactly zero
                s_nlse[buf][row] = ok ? boosted_row_term(lse) : -INFINITY;
                s_ndelta[buf][row] = ok ? -delta : 0.f;
            }
            if constexpr (FP4) {
                // the Q row's features (tid % 4) D / 4 .. + D / 4 - 1 as FP16
                uint8_t* dst = &s_q16[buf][(tid >> 2) * PITCH16 + 2 * (tid & 3) * (D / 4)];
#pragma unroll
                for (int q = 0; q < D / 32; ++q) {
                    const float sc = __builtin_amdgcn_cvt_f32_fp8((int)((nxt.q4s >> (8 * (q / 2))) & 0xff), 0);
                    *(h8*)(dst + 16 * q) = fp4x8_to_f16((uint32_t)nxt.q4[q], sc);
                }
            }
        };
        if (wave < 4) {
            fetch(jlo);
            stage(jlo);
        }
        // every load issued so far has landed (vmcnt(0)), so that inside the
        // loop only the prefetch of the next tile is outstanding
        wait_vm0_asm();
        __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();

        v16f dk[NDT], dv[NDT];
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) dk[i][v] = dv[i][v] = 0.f;

        // D = 128: the lane bases of the swizzled operand reads of the step
        // (Q rows of either query half and the transposed Q tile in buffer 0,
        // the wave's K rows), held across the loop; buffer 1 is 8 KB on, an
        // offset that commutes with the XOR addressing
        uint32_t qa0[2] = {0u, 0u}, ka0 = 0u, ta0 = 0u;
        if constexpr (CT::SWZ) {
#pragma unroll
            for (int t = 0; t < 2; ++t) qa0[t] = swz_row_addr(s_q[0], perm_row(t, lane & 31), lane);
            ka0 = swz_row_addr(s_kt, 32 * wave + (lane & 31), lane);
            ta0 = swz_tr_addr(s_q[0], lane);
        }
        constexpr uint32_t QBUF = sizeof(s_q[0]);
        // and of the dQ product's reads: the transposed K tile, the dS^ tile
        // (buffer 0)
        uint32_t kta0 = 0u, dsa0 = 0u;
        if constexpr (CT::SWZ) {
            kta0 = swz_tr_addr(s_kt, lane);
            dsa0 = lds_tr_addr(s_ds[0], SPITCH, lane);
        }
        constexpr uint32_t DSBUF = sizeof(s_ds[0]);

        // Tile j for the wave's keys: S, dP, P, dS, their codes (the k layout
        // of the dV / dK products: bytes 0-15 query half 0, 16-31 half 1), the
        // key-major dS^ rows of the tile's dQ product, then dV^T += dO^T P^ and
        // dK^T += Q^T dS^ over the tile's 64 queries.
        auto step = [&](int j) {
            // lane-derived offsets are recomputed in every step (an opaque
            // read of the thread index), not held across the loop next to the
            // dK / dV accumulators
            int lane = threadIdx.x;
            asm volatile("" : "+v"(lane));
            lane &= 63;
            const int g = lane >> 5;
            const int krow = 32 * wave + (lane & 31);
            const int kj = kw0 + (lane & 31);
            const bool kvalid = kj < e;
            const int pb = j & 1;
            const int qb = tile_base(j);
            const uint8_t* sq = s_q[pb];
            const uint8_t* sg = s_do[pb];
            v8i pc = {0, 0, 0, 0, 0, 0, 0, 0}, dc = pc;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                v4i pf = {0, 0, 0, 0}, df = {0, 0, 0, 0}, dr = {0, 0, 0, 0};
                int dse = 127;
                const bool active = wave_keys && (!a.causal || qb + 32 * t + 31 >= kw0);
                if (active) {
                    const int qr = perm_row(t, lane & 31);
                    // element v of lane group g is query qb + 32 t + 16 g + v.
                    // The dP product accumulates onto -D, so that pacc ends as
                    // dP - D without a subtraction per element.
                    v16f sacc, pacc;
#pragma unroll
                    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float4 x = *(const float4*)&s_ndelta[pb][32 * t + 16 * g + 4 * i];
                        pacc[4 * i] = x.x;
                        pacc[4 * i + 1] = x.y;
                        pacc[4 * i + 2] = x.z;
                        pacc[4 * i + 3] = x.w;
                    }
                    const int eqr = s_eq[pb][qr], edr = s_edo[pb][qr];
                    if constexpr (FP4) {
                        // S from the E2M1 views, expanded to exact FP16
#pragma unroll
                        for (int ks = 0; ks < NKH; ++ks)
                            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                *(const h8*)(s_q16[pb] + qr * PITCH16 + 2 * (16 * ks + 8 * g)), kh[ks], sacc, 0,
                                0, 0);
                    }
                    if constexpr (CT::SWZ) {
                        // Q / dO rows qr and K / V rows krow: one address per
                        // pair of tiles, the rest XOR and immediate offsets
                        const uint32_t qa = qa0[t] + pb * QBUF;
                        const uint32_t ka = ka0;
                        const int dqg = (int)(lds_addr(s_do[0]) - lds_addr(s_q[0]));
                        const int dkv = (int)(lds_addr(s_vt) - lds_addr(s_kt));
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) {
                            sacc = mfma_f8(swz_row_operand(qa, ks, 0), swz_row_operand(ka, ks, 0), sacc, eqr, ek);
                            pacc = mfma_f8(swz_row_operand(qa, ks, dqg), swz_row_operand(ka, ks, dkv), pacc, edr,
                                           ev);
                        }
                    } else {
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) {
                            if constexpr (!FP4)
                                sacc = mfma_f8(tile_row_operand<D>(sq, qr, 64 * ks, lane),
                                               tile_row_operand<D>(s_kt, krow, 64 * ks, lane), sacc, eqr, ek);
                            pacc = mfma_f8(tile_row_operand<D>(sg, qr, 64 * ks, lane),
                                           tile_row_operand<D>(s_vt, krow, 64 * ks, lane), pacc, edr, ev);
                        }
                    }
                    // keep the scheduler from hoisting the next operands above
                    // the element-wise work (register pressure)
                    __builtin_amdgcn_sched_barrier(0);
                    const float* nl = &s_nlse[pb][32 * t + 16 * g];
                    const bool full = kw0 + 32 <= e && (!a.causal || qb + 32 * t >= kw0 + 31);
                    float amax;
                    if (full) {
                        amax = softmax_grad_c<false>(sacc, pacc, nl, c2, 0);
                    } else {
                        const int lim = a.causal ? kj - qb - 32 * t - 16 * g : (kvalid ? -1 : 16);
                        amax = softmax_grad_c<true>(sacc, pacc, nl, c2, lim);
                    }
                    // block exponent of dS = that of 256 dS minus 8 (exact)
                    int et;
                    if constexpr (EXACT) {
                        // the dQ copy's per-row exponents: each query row's
                        // largest |256 dS| over the wave's 32 keys, one row per
                        // lane pair after a transpose-reduce, published in LDS as
                        // the dQ product's row scale and as the multiplier
                        // 2^(-e - 8) of the codes.  The exponent rule is
                        // monotone on non-zero maxima, so the block exponent is
                        // the largest row exponent over the non-zero rows (an
                        // all-zero row has exponent 0 and takes no part; an
                        // all-zero block has exponent 0).
                        const float rmax = row_absmax_transpose(pacc, lane);
                        const int erl = ceil_exp448(rmax * 0.00390625f);
                        if ((lane & 1) == 0) {
                            const int r = 32 * t + 16 * g + ((lane >> 1) & 15);
                            s_er[pb][wave][r] = erl + 127;
                            s_rm[pb][wave][r] = ldexpf(1.f, -erl - 8);
                        }
                        const int eb = (int)wave_max_u32(rmax == 0.f ? 0u : (uint32_t)(erl + 128));
                        et = eb == 0 ? 0 : eb - 128;
                    } else {
                        et = ceil_exp448(wave_max_nonneg(amax) * 0.00390625f);
                    }
                    dse = et + 127;
                    if constexpr (EXACT) {
                        // folded operands: P^ already carries 2^(e_dO - block
                        // max) (from the exponent term); dS x 2^(e_Q - block max)
                        // for dK (block exponent et); dS x 2^(e_K - block max)
                        // for dQ, coded against the row exponents (the
                        // conversion divides by 2^(block max - e_K))
                        const float* fq = &s_fq[pb][32 * t + 16 * g];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 f = *(const float4*)(fq + 4 * q);
                            pf[q] = (int)cvt4_fp8(sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]);
                            df[q] = (int)cvt4_fp8_div(pacc[4 * q] * f.x, pacc[4 * q + 1] * f.y, pacc[4 * q + 2] * f.z,
                                                      pacc[4 * q + 3] * f.w, ds_code_divisor(et));
                        }
                        const float* rm = &s_rm[pb][wave][32 * t + 16 * g];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 m = *(const float4*)(rm + 4 * q);
                            dr[q] = (int)cvt4_fp8_div(pacc[4 * q] * m.x, pacc[4 * q + 1] * m.y, pacc[4 * q + 2] * m.z,
                                                      pacc[4 * q + 3] * m.w, fkdiv);
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            pf[q] = (int)cvt4_fp8(sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]);
                            df[q] = (int)cvt4_fp8_div(pacc[4 * q], pacc[4 * q + 1], pacc[4 * q + 2],
                                                      pacc[4 * q + 3], ds_code_divisor(et));
                        }
                    }
                } else if constexpr (EXACT) {
                    if ((lane & 16) == 0) s_er[pb][wave][32 * t + 16 * g + (lane & 15)] = 127;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    pc[4 * t + q] = pf[q];
                    dc[4 * t + q] = df[q];
                }
                // the dQ product's key-major rows (per-token operands: the
                // K-folded copy with per-row exponents)
                *(v4i*)(s_ds[pb] + krow * SPITCH + 32 * t + 16 * g) = EXACT ? dr : df;
                if (lane == 0) s_dsexp[pb][t][wave] = dse;
            }
            __builtin_amdgcn_sched_barrier(0);
            if (wave_keys && (!a.causal || qb + 63 >= kw0)) {
                // the dS block exponents of this wave's key block, per query
                // half (lane group g supplies k block g's scale); the same
                // wave wrote them above
                const int dsg = s_dsexp[pb][g][wave];
                // per-token operands: the block maxima the fold factors are
                // relative to
                const int sdo = EXACT ? s_egb[pb][g] : s_edo[pb][32 * g];
                const int sqe = EXACT ? s_eqb[pb][g] : s_eq[pb][32 * g];
                if constexpr (CT::SWZ) {
                    const uint32_t ta = ta0 + pb * QBUF;
                    const int dqg = (int)(lds_addr(s_do[0]) - lds_addr(s_q[0]));
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        dv[dt] = mfma_f8(swz_tr_operand(ta, 0, dt, dqg), pc, dv[dt], sdo, kScaleMinus8);
                        dk[dt] = mfma_f8(swz_tr_operand(ta, 0, dt, 0), dc, dk[dt], sqe, dsg);
                    }
                } else {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        dv[dt] = mfma_f8(tile_tr_operand<D>(sg, 0, 32 * dt, lane), pc, dv[dt], sdo, kScaleMinus8);
                        dk[dt] = mfma_f8(tile_tr_operand<D>(sq, 0, 32 * dt, lane), dc, dk[dt], sqe, dsg);
                    }
                }
            }
        };

        // dQ of tile jp over the 256 keys: the 2 NDT output tiles of 32 x 32
        // (query half ct = ti / NDT, head-dim tile dt = ti % NDT), one per
        // wave (D = 128: all eight waves; D = 64: waves 4-7), each added to
        // the FP16 accumulator.  The row's prescale 2^(k_i + f) rides in the
        // A operand's block scale; the finalize applies 2^-(k_i + f) and the
        // rest of the softmax scale.
        auto dq = [&](int jp, int ti) {
            int lane = threadIdx.x;
            asm volatile("" : "+v"(lane));
            lane &= 63;
            const int g = lane >> 5;
            const int pb = jp & 1;
            const int qb = tile_base(jp), h = tile_head(jp);
            const int ct = ti / NDT, dt = ti % NDT;
            const int nrows = e - (qb + 32 * ct);
            if (nrows <= 0) return;
            const int qrow = 32 * ct + (lane & 31);
            const int kq = s_kq[jp % 3][qrow];
            v16f acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < NKEY / 64; ++ks) {
                // an item's first key is inside its document: the first block
                // always runs, so the zero accumulator is never needed
                if (ks > 0 && k0 + 64 * ks >= e) break;
                const int kb = 2 * ks + g;
                const int sa = min(max((EXACT ? s_er[pb][kb][qrow] : s_dsexp[pb][ct][kb]) + kq, 0), 254);
                if constexpr (CT::SWZ) {
                    const v8i kop = swz_tr_operand(kta0, 64 * ks, dt, 0);
                    const v8i dop = lds_tr_operand_at(dsa0 + pb * DSBUF + 64 * ks * SPITCH + 32 * ct, SPITCH);
                    acc = mfma_f8(dop, kop, acc, sa, s_ekb[kb]);
                } else {
                    const v8i kop = tile_tr_operand<D>(s_kt, 64 * ks, 32 * dt, lane);
                    acc = mfma_f8(lds_tr_operand(s_ds[pb] + 64 * ks * SPITCH, SPITCH, 0, 32 * ct, lane), kop, acc,
                                  sa, s_ekb[kb]);
                }
            }
            _Float16* tile = a.dq_acc + ((size_t)(qb + 32 * ct) * Hq + h) * D + 32 * dt;
            const uint32_t rs_bytes = (uint32_t)(Hq * D * 2);
            if (nrows >= 32) dq_tile_atomics_pk<false>(acc, tile, rs_bytes, lane, nrows);
            else dq_tile_atomics_pk<true>(acc, tile, rs_bytes, lane, nrows);
        };
        // D = 128: every wave owns one dQ output tile; waves 0-3 add theirs
        // after issuing the next tile's fetch, so that their final wait for
        // the fetch also covers atomics issued a whole step earlier
        constexpr bool DQ_ALL = NDT == 4;

        // both loops pass the same number of barriers
        if (wave < 4) {
            for (int j = jlo; j <= niter; ++j) {
                // fetch tile j + 1 (the last steps reload the last tile, unused)
                if (j + 1 < niter) fetch(j + 1);
                if constexpr (WITH_DQ && DQ_ALL) {
                    if (j > jlo) dq(j - 1, wave);
                }
                if (j < niter) step(j);
                if (j + 1 < niter) {
                    stage(j + 1);
                    // the direct loads count in vmcnt: they have landed once it
                    // is zero (an asm wait, which the compiler cannot drop: it
                    // does not count the asm loads)
                    if constexpr (DMA) {
                        wait_vm0_asm();
                        __builtin_amdgcn_s_waitcnt(0x0F70);
                    }
                }
                lds_barrier();
            }
        } else {
            // the reverse order of waves 0-3 (step first, then the dQ of the
            // previous tile, whose dS^ sits in the other buffer), so that the
            // two waves of a SIMD are in different phases: one's matrix
            // products overlap the other's element-wise work
            for (int j = jlo; j <= niter; ++j) {
                if (j < niter) step(j);
                if constexpr (WITH_DQ) {
                    if (j > jlo) dq(j - 1, DQ_ALL ? wave : wave - 4);
                }
                lds_barrier();
            }
        }

        // a split item: each half stores its raw accumulators in its slot
        // (16-byte chunk c of thread t at float4 index 512 c + t) and the
        // pair kernel, launched next, adds the two and writes the outputs
        if (half >= 0) {
            float4* mine = (float4*)a.dkv_part + (size_t)(2 * pair + half) * (8 * NDT) * 512;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    mine[(4 * dt + q) * 512 + tid] =
                        make_float4(dk[dt][4 * q], dk[dt][4 * q + 1], dk[dt][4 * q + 2], dk[dt][4 * q + 3]);
                    mine[(4 * NDT + 4 * dt + q) * 512 + tid] =
                        make_float4(dv[dt][4 * q], dv[dt][4 * q + 1], dv[dt][4 * q + 2], dv[dt][4 * q + 3]);
                }
        } else {
            store_dkdv<D>(a, dk, dv, kj, e, hk, lane);
        }
        // item boundary: every wave is done with this item's LDS before the next
        // item's first writes, and the next ticket is visible
        __syncthreads();
    }  // tickets
}

// The split items of the 256-key backward: workgroup p (512 threads, the
// thread layout of bwd_wide_kernel) adds the two halves' raw dK / dV
// accumulators of pair p = item x Hkv + kv head, slot 0 then slot 1, and
// writes the outputs.  The launch covers the most pairs the slots hold;
// workgroups past count[2] x Hkv return at once.
template <int D>
__global__ __launch_bounds__(512) void bwd_pair_kernel(AttnArgs a)
{
    constexpr int NDT = D / 32;
    constexpr int NC = 8 * NDT;  // float4 chunks of dk, then dv, per thread
    const int pair = blockIdx.x;
    if (pair >= a.count[2] * a.Hkv) return;
    const int item = pair / a.Hkv, hk = pair % a.Hkv;
    const int b = a.items[2 * item], kt = a.items[2 * item + 1];
    const int e = a.cu[b + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int kj = a.cu[b] + 256 * kt + 32 * wave + (lane & 31);
    const float4* s0 = (const float4*)a.dkv_part + (size_t)(2 * pair) * NC * 512;
    const float4* s1 = s0 + (size_t)NC * 512;
    v16f dk[NDT], dv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ck = (4 * dt + q) * 512 + tid, cv = (4 * NDT + 4 * dt + q) * 512 + tid;
            const float4 x0 = s0[ck], x1 = s1[ck], y0 = s0[cv], y1 = s1[cv];
            dk[dt][4 * q] = x0.x + x1.x;
            dk[dt][4 * q + 1] = x0.y + x1.y;
            dk[dt][4 * q + 2] = x0.z + x1.z;
            dk[dt][4 * q + 3] = x0.w + x1.w;
            dv[dt][4 * q] = y0.x + y1.x;
            dv[dt][4 * q + 1] = y0.y + y1.y;
            dv[dt][4 * q + 2] = y0.z + y1.z;
            dv[dt][4 * q + 3] = y0.w + y1.w;
        }
    store_dkdv<D>(a, dk, dv, kj, e, hk, lane);
}

// Query-major dQ for the deterministic backward: a workgroup (4 waves x 32
// queries) owns a 128-query tile of one document and one q head and walks
// the visible keys in 64-key steps, recomputing S and dP exactly as the
// key-major kernel does but with lanes on queries (S^T = K Q^T with the key
// rows permuted).  dS^ then already sits in registers in the k layout of the
// dQ^T = K^T dS^T MFMA, and dQ accumulates in FP32 registers in a fixed
// order: no atomics, bitwise repeatable.  The 32 x 32 dS blocks (the wave's
// 32 queries x 32 keys) and their exponents are the same as in the key-major
// kernel.
struct KVStep {
    v4i k[2], v[2];
    int ek, ev;
};

template <int D>
__device__ __forceinline__ void load_kvstep(const AttnArgs& a, KVStep& r, int hk, int kt0, int e,
                                            int tid)
{
    constexpr int CPR = D / 16;
    const int Hkv = a.Hkv;
    const size_t T = (size_t)a.T;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int c = tid + 256 * k;
        const int row = c / CPR, col = 16 * (c % CPR);
        const int t = kt0 + row;
        r.k[k] = v4i{0, 0, 0, 0};
        r.v[k] = v4i{0, 0, 0, 0};
        if (row < 64 && t < e) {
            r.k[k] = *(const v4i*)(a.k_codes + ((size_t)t * Hkv + hk) * D + col);
            r.v[k] = *(const v4i*)(a.v_codes + ((size_t)t * Hkv + hk) * D + col);
        }
    }
    r.ek = 127;
    r.ev = 127;
    if (tid < 64) {
        const int t = kt0 + tid;
        if (t < e) {
            r.ek = (int)a.k_exps[(size_t)hk * T + t];
            r.ev = (int)a.v_exps[(size_t)hk * T + t];
        }
    }
}

template <int D>
// Two workgroups per CU (two waves per SIMD): at d = 128 the kernel fits 244
// VGPRs without spilling; with one wave per SIMD it had no latency hiding
// and ran at less than half the speed.
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(AttnArgs a)
{
    constexpr int PITCH = D + 16;
    constexpr int NKS = D / 64;
    constexpr int NDT = D / 32;
    constexpr int CPR = D / 16;
    __shared__ __attribute__((aligned(16))) uint8_t s_k[2][64 * PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[2][64 * PITCH];
    __shared__ int s_ek[2][64], s_ev[2][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), g = lane >> 5;
    const int Hq = a.Hq, Hkv = a.Hkv;
    const size_t T = (size_t)a.T;
    // kv heads first within an item: the q heads sharing a kv head run on one
    // XCD (workgroup i runs on XCD i % 8) and share its L2 copy of K/V
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

    // Q and dO rows of this lane's query: B operands of S^T and dP^T
    v8i qf[NKS], gf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (qvalid) {
            qf[ks] = row_operand(a.q_codes + ((size_t)qi * Hq + h) * D + 64 * ks, lane);
            gf[ks] = row_operand(a.do_codes + ((size_t)qi * Hq + h) * D + 64 * ks, lane);
        } else {
            qf[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            gf[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    const int eq = qvalid ? (int)a.q_exps[(size_t)h * T + qi] : 127;
    const int edo = qvalid ? (int)a.do_exps[(size_t)h * T + qi] : 127;
    // 256 P = exp2(s c2 + 8 - LSE log2 e), formed as in the key-major kernel
    const float nl = qvalid ? boosted_row_term(a.lse_in[(size_t)h * T + qi]) : -INFINITY;
    const float delta = qvalid ? a.delta[(size_t)h * T + qi] : 0.f;

    const int kend = a.causal ? min(q0 + 128, e) : e;
    const int nsteps = (kend - s + 63) / 64;
    const int kend_w = a.causal ? min(qw + 32, e) : e;

    v16f dq[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) dq[dt][v] = 0.f;

    auto stage = [&](const KVStep& t, int buf) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int c = tid + 256 * k;
            const int row = c / CPR, col = 16 * (c % CPR);
            if (row < 64) {
                *(v4i*)(&s_k[buf][row * PITCH + col]) = t.k[k];
                *(v4i*)(&s_v[buf][row * PITCH + col]) = t.v[k];
            }
        }
        if (tid < 64) {
            s_ek[buf][tid] = t.ek;
            s_ev[buf][tid] = t.ev;
        }
    };

    KVStep nxt;
    if (nsteps > 0) {
        load_kvstep<D>(a, nxt, hk, s, e, tid);
        stage(nxt, 0);
    }
    lds_barrier();

    for (int st = 0; st < nsteps; ++st) {
        const int cur = st & 1;
        const int kt0 = s + 64 * st;
        const bool more = st + 1 < nsteps;
        if (more) load_kvstep<D>(a, nxt, hk, kt0 + 64, e, tid);
        if (kt0 < kend_w) {
            const uint8_t* sk = s_k[cur];
            const uint8_t* sv = s_v[cur];
            v16f sacc[2], pacc[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int krow = perm_row(t, lane & 31);
                // the dP product accumulates onto -D (lane = query), as in the
                // key-major kernel, so both form dP - D the same way
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    sacc[t][v] = 0.f;
                    pacc[t][v] = -delta;
                }
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    sacc[t] = mfma_f8(row_operand(sk + krow * PITCH + 64 * ks, lane), qf[ks],
                                      sacc[t], s_ek[cur][krow], eq);
                    pacc[t] = mfma_f8(row_operand(sv + krow * PITCH + 64 * ks, lane), gf[ks],
                                      pacc[t], s_ev[cur][krow], edo);
                }
            }
            // element (t, v) of lane group g <-> key kt0 + 32 t + 16 g + v
            float amax[2] = {0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = kt0 + 32 * t + 16 * g + v;
                    const bool vis = qvalid && key < e && (!a.causal || key <= qi);
                    const float p = vis ? __builtin_amdgcn_exp2f(fmaf(sacc[t][v], c2, nl)) : 0.f;
                    const float ds = p * pacc[t][v];  // 256 dS
                    pacc[t][v] = ds;
                    amax[t] = fmaxf(amax[t], fabsf(ds));
                }
            int dse[2];
            v8i df;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // block exponent of dS = that of 256 dS minus 8 (exact), and the
                // codes of 256 dS over 2^(et + 8), as in the key-major kernel
                const int et = ceil_exp448(wave_max_nonneg(amax[t]) * 0.00390625f);
                dse[t] = et + 127;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    df[4 * t + q] = (int)cvt4_fp8_div(pacc[t][4 * q], pacc[t][4 * q + 1], pacc[t][4 * q + 2],
                                                      pacc[t][4 * q + 3], ds_code_divisor(et));
            }
            // dQ^T += K^T dS^T: K read k-major from the token-major LDS tile
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                dq[dt] = mfma_f8(lds_tr_operand(sk, PITCH, 0, 32 * dt, lane), df, dq[dt],
                                 s_ek[cur][32 * g], dse[g]);
        }
        if (more) stage(nxt, cur ^ 1);
        lds_barrier();
    }

    if (qvalid) {
        uint16_t* row = a.dq + ((size_t)qi * Hq + h) * D;
        const float sc = a.scale;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v2i w;
                w.x = (int)pack_bf16x2(dq[dt][4 * q] * sc, dq[dt][4 * q + 1] * sc);
                w.y = (int)pack_bf16x2(dq[dt][4 * q + 2] * sc, dq[dt][4 * q + 3] * sc);
                *(v2i*)(row + 32 * dt + 8 * q + 4 * g) = w;
            }
    }
}

// dQ = acc * (scale 2^-f) * 2^-k_i -> bf16 for every row, the accumulator
// holding 2^(k_i + f) sum dS^ K^ (2^f <= scale < 2^(f + 1)); dK = dV = 0 on
// padding rows.
template <int D, bool FROM_ACC>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(AttnArgs a)
{
    const int ntok = a.cu[a.B];
    const size_t T = (size_t)a.T;
    const size_t nq = T * a.Hq * (D / 8);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nq; i += (size_t)gridDim.x * 256) {
        const size_t row = i / (D / 8);
        const int c = (int)(i % (D / 8));
        const int t = (int)(row / a.Hq), h = (int)(row % a.Hq);
        if constexpr (FROM_ACC) {
            const float f = ldexpf(a.scale_res, -(int)a.prescale[(size_t)h * T + t]);
            const h8 raw = *(const h8*)(a.dq_acc + row * D + 8 * c);
            float y[8] = {(float)raw.s0 * f, (float)raw.s1 * f, (float)raw.s2 * f, (float)raw.s3 * f,
                          (float)raw.s4 * f, (float)raw.s5 * f, (float)raw.s6 * f, (float)raw.s7 * f};
            // rotated Q and K: dQ = dQ_r H (a row is D / 8 consecutive lanes:
            // the stride keeps every lane on the same chunk c)
            if (a.rotate) fwht_row<D>(y, threadIdx.x & 63);
            v4i out;
            out.x = (int)pack_bf16x2(y[0], y[1]);
            out.y = (int)pack_bf16x2(y[2], y[3]);
            out.z = (int)pack_bf16x2(y[4], y[5]);
            out.w = (int)pack_bf16x2(y[6], y[7]);
            *(v4i*)(a.dq + row * D + 8 * c) = out;
        } else if (t >= ntok) {
            *(v4i*)(a.dq + row * D + 8 * c) = v4i{0, 0, 0, 0};
        }
        if (row < T * a.Hkv) {
            const int t2 = (int)(row / a.Hkv);
            if (t2 >= ntok) {
                *(v4i*)(a.dk + row * D + 8 * c) = v4i{0, 0, 0, 0};
                *(v4i*)(a.dv + row * D + 8 * c) = v4i{0, 0, 0, 0};
            }
        }
    }
}

}  // namespace

hipError_t launch_bwd(const AttnArgs& a, int D, int max_items, bool with_dq, hipStream_t stream)
{
    if (max_items <= 0) return hipSuccess;
    // persistent grid: as many workgroups as the device holds at once (one per
    // CU at this kernel's register and LDS use), never more than the tickets
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        return hipErrorInvalidDevice;
    const dim3 grid((unsigned)std::min<int64_t>((int64_t)max_items * a.Hkv, ncu));
#define FLAMIA_BWD(DD, WQ, MM) \
    FLAMIA_LAUNCH((bwd_kernel<DD, WQ, MM>), grid, dim3(512), stream, a.ev_start, a.ev_stop, a)
    if (D == 128) {
        if (a.mode == MODE_EXACT) {
            if (with_dq) FLAMIA_BWD(128, true, MODE_EXACT);
            else FLAMIA_BWD(128, false, MODE_EXACT);
        } else {
            if (with_dq) FLAMIA_BWD(128, true, MODE_BLOCK);
            else FLAMIA_BWD(128, false, MODE_BLOCK);
        }
    } else {
        if (a.mode == MODE_FP4) {
            if (with_dq) FLAMIA_BWD(64, true, MODE_FP4);
            else FLAMIA_BWD(64, false, MODE_FP4);
        } else if (a.mode == MODE_EXACT) {
            if (with_dq) FLAMIA_BWD(64, true, MODE_EXACT);
            else FLAMIA_BWD(64, false, MODE_EXACT);
        } else {
            if (with_dq) FLAMIA_BWD(64, true, MODE_BLOCK);
            else FLAMIA_BWD(64, false, MODE_BLOCK);
        }
    }
#undef FLAMIA_BWD
    return hipGetLastError();
}

int bwd_wide_workgroups(int64_t tickets)
{
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        return 0;
    return (int)std::min<int64_t>(tickets, ncu);
}

hipError_t launch_bwd_wide(const AttnArgs& a, int D, int max_items, bool with_dq, hipStream_t stream)
{
    if (max_items <= 0) return hipSuccess;
    // split items add up to one more ticket per item and kv head
    const int wgs = bwd_wide_workgroups(2 * (int64_t)max_items * a.Hkv);
    if (wgs <= 0) return hipErrorInvalidDevice;
    const dim3 grid((unsigned)wgs);
#define FLAMIA_BWDW(DD, WQ, MM) \
    FLAMIA_LAUNCH((bwd_wide_kernel<DD, WQ, MM>), grid, dim3(512), stream, a.ev_start, a.ev_stop, a)
    if (a.mode != MODE_BLOCK) {
        // per-token operands: d = 64, dQ by atomics (no deterministic form)
        if (D != 64 || !with_dq) return hipErrorInvalidValue;
        if (a.mode == MODE_FP4) FLAMIA_BWDW(64, true, MODE_FP4);
        else FLAMIA_BWDW(64, true, MODE_EXACT);
    } else if (D == 128) {
        if (with_dq) FLAMIA_BWDW(128, true, MODE_BLOCK);
        else FLAMIA_BWDW(128, false, MODE_BLOCK);
    } else {
        if (with_dq) FLAMIA_BWDW(64, true, MODE_BLOCK);
        else FLAMIA_BWDW(64, false, MODE_BLOCK);
    }
#undef FLAMIA_BWDW
    return hipGetLastError();
}

hipError_t launch_bwd_pairs(const AttnArgs& a, int D, int max_pairs, hipStream_t stream)
{
    if (max_pairs <= 0) return hipSuccess;
    if (D == 128) hipLaunchKernelGGL(bwd_pair_kernel<128>, dim3(max_pairs), dim3(512), 0, stream, a);
    else hipLaunchKernelGGL(bwd_pair_kernel<64>, dim3(max_pairs), dim3(512), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const AttnArgs& a, int D, int max_items, hipStream_t stream)
{
    if (max_items <= 0) return hipSuccess;
    const dim3 grid((unsigned)max_items * a.Hq);
    if (D == 128) hipLaunchKernelGGL(bwd_dq_kernel<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(bwd_dq_kernel<64>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_finalize(const AttnArgs& a, int D, bool dq_from_acc, hipStream_t stream)
{
    if (a.T == 0) return hipSuccess;
    const size_t n = (size_t)a.T * a.Hq * (D / 8);
    const unsigned blocks = (unsigned)min((size_t)8192, (n + 255) / 256);
    if (D == 128) {
        if (dq_from_acc) hipLaunchKernelGGL((bwd_finalize_kernel<128, true>), dim3(blocks), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((bwd_finalize_kernel<128, false>), dim3(blocks), dim3(256), 0, stream, a);
    } else {
        if (dq_from_acc) hipLaunchKernelGGL((bwd_finalize_kernel<64, true>), dim3(blocks), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((bwd_finalize_kernel<64, false>), dim3(blocks), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace flamia
