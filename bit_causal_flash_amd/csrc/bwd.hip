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
// Tiling: a workgroup (4 waves) owns a document-local 128-key tile of one kv
// head (wave w: 32 keys, one token block) and loops over the q heads of its
// group and the 64-query tiles that can see its keys; dK and dV accumulate
// in registers across all of them (GQA head reduction without atomics).  S and
// dP are computed with the query rows permuted so the accumulators already
// hold P^ and dS^ in the k layout of the dV / dK MFMAs.  Q, dO and K are
// staged token-major in LDS and read k-major with ds_read_b64_tr_b8 where the
// contraction runs over tokens: one copy of every code tensor serves both
// orientations.  dS^ goes through LDS once, transposed, for dQ.
#include "device.hpp"
#include "kernels.hpp"

namespace flamia {

namespace {

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_kernel(AttnArgs a)
{
    constexpr int PITCH = D + 16;
    constexpr int SPITCH = 128 + 16;
    constexpr int NKS = D / 64;
    constexpr int NDT = D / 32;
    constexpr int CPR = D / 16;
    __shared__ __attribute__((aligned(16))) uint8_t s_kt[128 * PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[64 * PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_do[64 * PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_ds[64 * SPITCH];
    __shared__ int s_eq[64], s_edo[64];
    __shared__ float s_lse2[64], s_delta[64], s_qscale[64];
    __shared__ int s_dsexp[2][4];
    __shared__ int s_ekb[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
    const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
    const size_t T = (size_t)a.T;
    const int item = blockIdx.x / Hkv, hk = blockIdx.x % Hkv;
    if (item >= *a.count) return;
    const int b = a.items[2 * item], kt = a.items[2 * item + 1];
    const int s = a.cu[b], e = a.cu[b + 1];
    const int k0 = s + 128 * kt;
    const int kw0 = k0 + 32 * wave;
    const int kj = kw0 + (lane & 31);
    const bool kvalid = kj < e;
    const bool wave_keys = kw0 < e;
    const float c2 = a.c2;

    // the workgroup's K tile, token-major, for the dQ MFMA (k = keys)
    for (int c = tid; c < 128 * CPR; c += 256) {
        const int row = c / CPR, col = 16 * (c % CPR);
        const int t = k0 + row;
        v4i kv = {0, 0, 0, 0};
        if (t < e) kv = *(const v4i*)(a.k_codes + ((size_t)t * Hkv + hk) * D + col);
        *(v4i*)(s_kt + row * PITCH + col) = kv;
    }
    if (tid < 4) s_ekb[tid] = (k0 + 32 * tid < e) ? (int)a.k_exps[(size_t)hk * T + k0 + 32 * tid] : 127;

    // this wave's K and V rows: B operands of S = Q K^T and dP = dO V^T
    v8i kf[NKS], vf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        if (kvalid) {
            kf[ks] = row_operand(a.k_codes + ((size_t)kj * Hkv + hk) * D + 64 * ks, lane);
            vf[ks] = row_operand(a.v_codes + ((size_t)kj * Hkv + hk) * D + 64 * ks, lane);
        } else {
            kf[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            vf[ks] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    const int ek = kvalid ? (int)a.k_exps[(size_t)hk * T + kj] : 127;
    const int ev = kvalid ? (int)a.v_exps[(size_t)hk * T + kj] : 127;

    v16f dk[NDT], dv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) dk[dt][v] = dv[dt][v] = 0.f;

    const int qt_lo = a.causal ? 2 * kt : 0;
    const int qt_hi = (e - s + 63) / 64;
    for (int hh = 0; hh < G; ++hh) {
        const int h = hk * G + hh;
        for (int qt = qt_lo; qt < qt_hi; ++qt) {
            const int qb = s + 64 * qt;
            __syncthreads();
            for (int c = tid; c < 64 * CPR; c += 256) {
                const int row = c / CPR, col = 16 * (c % CPR);
                const int t = qb + row;
                v4i qv = {0, 0, 0, 0}, gv = {0, 0, 0, 0};
                if (t < e) {
                    qv = *(const v4i*)(a.q_codes + ((size_t)t * Hq + h) * D + col);
                    gv = *(const v4i*)(a.do_codes + ((size_t)t * Hq + h) * D + col);
                }
                *(v4i*)(s_q + row * PITCH + col) = qv;
                *(v4i*)(s_do + row * PITCH + col) = gv;
            }
            if (tid < 64) {
                const int t = qb + tid;
                const bool ok = t < e;
                s_eq[tid] = ok ? (int)a.q_exps[(size_t)h * T + t] : 127;
                s_edo[tid] = ok ? (int)a.do_exps[(size_t)h * T + t] : 127;
                s_lse2[tid] = ok ? a.lse_in[(size_t)h * T + t] * kLog2e : INFINITY;
                s_delta[tid] = ok ? a.delta[(size_t)h * T + t] : 0.f;
                s_qscale[tid] = ok ? ldexpf(a.scale, (int)a.prescale[(size_t)h * T + t]) : 0.f;
            }
            __syncthreads();

            const bool active = wave_keys && (!a.causal || qb + 63 >= kw0);
            v8i pf = {0, 0, 0, 0, 0, 0, 0, 0}, df = {0, 0, 0, 0, 0, 0, 0, 0};
            int dse[2] = {127, 127};
            if (active) {
                v16f sacc[2], pacc[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int qr = perm_row(t, lane & 31);
#pragma unroll
                    for (int v = 0; v < 16; ++v) sacc[t][v] = pacc[t][v] = 0.f;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        sacc[t] = mfma_f8(row_operand(s_q + qr * PITCH + 64 * ks, lane), kf[ks],
                                          sacc[t], s_eq[qr], ek);
                        pacc[t] = mfma_f8(row_operand(s_do + qr * PITCH + 64 * ks, lane), vf[ks],
                                          pacc[t], s_edo[qr], ev);
                    }
                }
                // P, dS; element (t, v) of lane group g <-> query 32 t + 16 g + v
                float amax[2] = {0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int qq = 32 * t + 16 * g + v;
                        const int qi = qb + qq;
                        const bool vis = kvalid && qi < e && (!a.causal || kj <= qi);
                        const float p =
                            vis ? __builtin_amdgcn_exp2f(fmaf(sacc[t][v], c2, -s_lse2[qq])) : 0.f;
                        const float ds = p * (pacc[t][v] - s_delta[qq]);
                        sacc[t][v] = p;
                        pacc[t][v] = ds;
                        amax[t] = fmaxf(amax[t], fabsf(ds));
                    }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int et = ceil_exp448(wave_max(amax[t]));
                    dse[t] = et + 127;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        pf[4 * t + q] = (int)cvt4_fp8(fminf(256.f * sacc[t][4 * q], 448.f),
                                                      fminf(256.f * sacc[t][4 * q + 1], 448.f),
                                                      fminf(256.f * sacc[t][4 * q + 2], 448.f),
                                                      fminf(256.f * sacc[t][4 * q + 3], 448.f));
                        df[4 * t + q] = (int)cvt4_fp8(
                            ldexpf(pacc[t][4 * q], -et), ldexpf(pacc[t][4 * q + 1], -et),
                            ldexpf(pacc[t][4 * q + 2], -et), ldexpf(pacc[t][4 * q + 3], -et));
                    }
                }
                // dV^T += dO^T P^ and dK^T += Q^T dS^ (k = the tile's 64 queries)
                const int sdo = s_edo[32 * g];
                const int sq = s_eq[32 * g];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    dv[dt] = mfma_f8(lds_tr_operand(s_do, PITCH, 0, 32 * dt, lane), pf, dv[dt], sdo,
                                     kScaleMinus8);
                    dk[dt] = mfma_f8(lds_tr_operand(s_q, PITCH, 0, 32 * dt, lane), df, dk[dt], sq,
                                     dse[g]);
                }
            }

            // dS^ to LDS, query-major, for the dQ product
            {
                const int kcol = 32 * wave + (lane & 31);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const uint32_t w = (uint32_t)df[4 * t + v / 4];
                        s_ds[(32 * t + 16 * g + v) * SPITCH + kcol] = (uint8_t)(w >> (8 * (v % 4)));
                    }
                if (lane == 0) {
                    s_dsexp[0][wave] = dse[0];
                    s_dsexp[1][wave] = dse[1];
                }
            }
            __syncthreads();

            // dQ^T = K^T dS^T over the tile's 128 keys, 32 x 32 output tiles
            for (int j = wave; j < 2 * NDT; j += 4) {
                const int dt = j % NDT, ct = j / NDT;
                if (qb + 32 * ct >= e) continue;
                if (a.causal && qb + 32 * ct + 31 < k0) continue;
                const int qcol = 32 * ct + (lane & 31);
                v16f acc;
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (k0 + 64 * ks >= e) break;
                    acc = mfma_f8(lds_tr_operand(s_kt + 64 * ks * PITCH, PITCH, 0, 32 * dt, lane),
                                  row_operand(s_ds + qcol * SPITCH + 64 * ks, lane), acc,
                                  s_ekb[2 * ks + g], s_dsexp[ct][2 * ks + g]);
                }
                const int qi = qb + qcol;
                if (qi < e) {
                    const float f = s_qscale[qcol];
                    _Float16* dst = a.dq_acc + ((size_t)qi * Hq + h) * D + 32 * dt + 4 * g;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int pr = 0; pr < 2; ++pr) {
                            h2 val;
                            val.x = (_Float16)(acc[4 * q + 2 * pr] * f);
                            val.y = (_Float16)(acc[4 * q + 2 * pr + 1] * f);
                            __builtin_amdgcn_global_atomic_fadd_v2f16((h2*)(dst + 8 * q + 2 * pr),
                                                                      val);
                        }
                }
            }
        }
    }

    if (kvalid) {
        uint16_t* krow = a.dk + ((size_t)kj * Hkv + hk) * D;
        uint16_t* vrow = a.dv + ((size_t)kj * Hkv + hk) * D;
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
                *(v2i*)(krow + 32 * dt + 8 * q + 4 * g) = wk;
                *(v2i*)(vrow + 32 * dt + 8 * q + 4 * g) = wv;
            }
    }
}

// dQ = acc * 2^-k_i -> bf16 for every row; dK = dV = 0 on padding rows.
template <int D>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(AttnArgs a)
{
    const int ntok = a.cu[a.B];
    const size_t T = (size_t)a.T;
    const size_t nq = T * a.Hq * (D / 8);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nq; i += (size_t)gridDim.x * 256) {
        const size_t row = i / (D / 8);
        const int c = (int)(i % (D / 8));
        const int t = (int)(row / a.Hq), h = (int)(row % a.Hq);
        const int k = (int)a.prescale[(size_t)h * T + t];
        const h8 raw = *(const h8*)(a.dq_acc + row * D + 8 * c);
        v4i out;
        out.x = (int)pack_bf16x2(ldexpf((float)raw.s0, -k), ldexpf((float)raw.s1, -k));
        out.y = (int)pack_bf16x2(ldexpf((float)raw.s2, -k), ldexpf((float)raw.s3, -k));
        out.z = (int)pack_bf16x2(ldexpf((float)raw.s4, -k), ldexpf((float)raw.s5, -k));
        out.w = (int)pack_bf16x2(ldexpf((float)raw.s6, -k), ldexpf((float)raw.s7, -k));
        *(v4i*)(a.dq + row * D + 8 * c) = out;
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

hipError_t launch_bwd(const AttnArgs& a, int D, int max_items, hipStream_t stream)
{
    if (max_items <= 0) return hipSuccess;
    const dim3 grid((unsigned)max_items * a.Hkv);
    if (D == 128) hipLaunchKernelGGL(bwd_kernel<128>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(bwd_kernel<64>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_bwd_finalize(const AttnArgs& a, int D, hipStream_t stream)
{
    if (a.T == 0) return hipSuccess;
    const size_t n = (size_t)a.T * a.Hq * (D / 8);
    const unsigned blocks = (unsigned)min((size_t)8192, (n + 255) / 256);
    if (D == 128) hipLaunchKernelGGL(bwd_finalize_kernel<128>, dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(bwd_finalize_kernel<64>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace flamia
