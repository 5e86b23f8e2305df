// quant.hip -- document-local token-block E4M3 quantizer, and the backward
// preparation that quantizes dO with the same rule while computing
// D_i = dO^_i . O_i and the causal dQ prescale exponent.
//
// Method: FLAMIA review section 3 (one power-of-two exponent per
// document-local block of <= 32 tokens x the full head dim), section 4 (the
// conservative exponent: the smallest e with amax / 2^e <= 448; zero blocks
// take e = 0), section 5 Algorithm 1 step 09 ("encode G once; compute D from
// reconstructed G and saved O") and section 4 "Forward locality and backward
// locality differ" (the dQ accumulator scale must come from the row's own dO
// and the running maxima of the visible K and V magnitudes).
//
// Work decomposition: one workgroup per (32-token window, head).  It owns
// every document-local block whose first token lies in the window, so it
// touches at most 63 rows and every token is read exactly once; it also
// writes the padding rows (t >= cu[B]) of its window.  The kernel is
// HBM-bound: 2 bytes read and 1 byte written per element (plus 2 bytes of O
// read, 2 bytes of accumulator zeroing and 5 bytes per row for the backward
// preparation).
#include "device.hpp"
#include "kernels.hpp"

namespace flamia {

namespace {

template <int D, bool PREP>
__global__ __launch_bounds__(256) void quant_kernel(QuantArgs a)
{
    constexpr int TPR = D / 8;            // threads per row (16 bytes of bf16 each)
    constexpr int RPP = 256 / TPR;        // rows per pass
    constexpr int NPASS = 64 / RPP;       // passes covering 64 local rows
    const int tid = threadIdx.x;
    const int w0 = 32 * blockIdx.x;       // window start
    const int h = blockIdx.y;
    const int H = a.H, T = a.T, B = a.B;
    const int32_t* __restrict__ cu = a.cu;
    const int ntok = cu[B];

    __shared__ int s_bs[64], s_be[64];    // block start / end of local row (or -1)
    __shared__ float s_rowmax[64];
    __shared__ int s_exp[64];
    __shared__ float s_rowdot[64];
    __shared__ int s_rownz[64];
    __shared__ int s_pref[64];            // prefix max of V + K exponents (PREP)

    if (tid < 64) {
        const int t = w0 + tid;
        int bs = -1, be = -1;
        if (t < ntok && t < T) {
            const int b = doc_of(cu, B, t);
            const int s = cu[b], e = cu[b + 1];
            const int blk = a.block;
            const int start = s + blk * ((t - s) / blk);
            if (start >= w0 && start < w0 + 32) {
                bs = start;
                be = min(start + blk, e);
            }
        }
        s_bs[tid] = bs;
        s_be[tid] = be;
        s_rowdot[tid] = 0.f;
        s_rownz[tid] = 0;
    }
    __syncthreads();

    // load rows and their row maxima
    const int chunk = tid % TPR;
    float xv[NPASS][8];
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int r = p * RPP + tid / TPR;
        const int t = w0 + r;
        float m = 0.f;
        if (s_bs[r] >= 0) {
            const v4i raw = *(const v4i*)(a.x + ((size_t)t * H + h) * D + 8 * chunk);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                xv[p][2 * k] = bf16_to_f32((uint16_t)(raw[k] & 0xffff));
                xv[p][2 * k + 1] = bf16_to_f32((uint16_t)((uint32_t)raw[k] >> 16));
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(xv[p][k]));
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) xv[p][k] = 0.f;
        }
#pragma unroll
        for (int o = TPR / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        if (chunk == 0) s_rowmax[r] = m;
    }
    __syncthreads();

    // block exponent, per local row
    if (tid < 64) {
        int e = 0;
        if (s_bs[tid] >= 0) {
            const int lo = s_bs[tid] - w0, hi = s_be[tid] - w0;
            float amax = 0.f;
            for (int r = lo; r < hi; ++r) amax = fmaxf(amax, s_rowmax[r]);
            e = ceil_exp448(amax);
        }
        s_exp[tid] = e;
        const int t = w0 + tid;
        if (t < T && (s_bs[tid] >= 0 || (t >= ntok && tid < 32)))
            a.exps[(size_t)h * T + t] = (uint8_t)(e + 127);
    }

    if constexpr (PREP) {
        // prefix maxima of V and K block exponents over the keys row i may
        // see, for every block that starts in this window: one workgroup-wide
        // reduction per block (usually one block per window)
        __shared__ int s_red[2][256];
        const int g = h * a.Hkv / H;
        for (int r0 = 0; r0 < 32; ++r0) {
            if (s_bs[r0] != w0 + r0) continue;  // uniform across the workgroup
            const int t0 = w0 + r0;
            const int b = doc_of(cu, B, t0);
            const int s = cu[b], e = cu[b + 1];
            const int blk = a.block;
            const int last = a.causal ? min(s_be[r0], e) : e;  // exclusive key end
            const int nb = (last - s + blk - 1) / blk;
            int mv = -1000, mk = -1000;
            for (int kb = tid; kb < nb; kb += 256) {
                const int j = s + kb * blk;
                mv = max(mv, (int)a.v_exps[(size_t)g * T + j] - 127);
                mk = max(mk, (int)a.k_exps[(size_t)g * T + j] - 127);
            }
            s_red[0][tid] = mv;
            s_red[1][tid] = mk;
            __syncthreads();
            for (int o = 128; o >= 1; o >>= 1) {
                if (tid < o) {
                    s_red[0][tid] = max(s_red[0][tid], s_red[0][tid + o]);
                    s_red[1][tid] = max(s_red[1][tid], s_red[1][tid + o]);
                }
                __syncthreads();
            }
            if (tid == 0) s_pref[r0] = s_red[0][0] + s_red[1][0];
            __syncthreads();
        }
    }
    __syncthreads();

    // codes (and, for the backward preparation, D and the accumulator zeros)
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
        const int r = p * RPP + tid / TPR;
        const int t = w0 + r;
        if (t >= T) continue;
        const size_t off = ((size_t)t * H + h) * D + 8 * chunk;
        const bool mine = s_bs[r] >= 0;
        const bool pad = (t >= ntok) && r < 32;
        if (!mine && !pad) continue;
        uint32_t lo = 0, hi = 0;
        float dot = 0.f;
        if (mine) {
            const int e = s_exp[r];
            float y[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = ldexpf(xv[p][k], -e);
            lo = cvt4_fp8(y[0], y[1], y[2], y[3]);
            hi = cvt4_fp8(y[4], y[5], y[6], y[7]);
            if constexpr (PREP) {
                const v4i oraw = *(const v4i*)(a.o + off);
                v2f d0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
                v2f d1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
                v2f d2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
                v2f d3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
                const float dq[8] = {d0.x, d0.y, d1.x, d1.y, d2.x, d2.y, d3.x, d3.y};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    dot += ldexpf(dq[2 * k], e) * bf16_to_f32((uint16_t)(oraw[k] & 0xffff));
                    dot += ldexpf(dq[2 * k + 1], e) * bf16_to_f32((uint16_t)((uint32_t)oraw[k] >> 16));
                }
            }
        }
        v2i cw;
        cw.x = (int)lo;
        cw.y = (int)hi;
        *(v2i*)(a.codes + off) = cw;
        if constexpr (PREP) {
            // zero this row's FP16 dQ accumulator chunk
            v4i z = {0, 0, 0, 0};
            *(v4i*)(a.dq_acc + off) = z;
            const int nz = ((lo | hi) & 0x7f7f7f7fu) != 0;
#pragma unroll
            for (int o = TPR / 2; o >= 1; o >>= 1) {
                dot += __shfl_xor(dot, o, kWave);
            }
            if (nz) atomicOr(&s_rownz[r], 1);
            if (chunk == 0) s_rowdot[r] = dot;
        }
    }

    if constexpr (PREP) {
        __syncthreads();
        if (tid < 64) {
            const int t = w0 + tid;
            if (t < T && (s_bs[tid] >= 0 || (t >= ntok && tid < 32))) {
                int k = 0;
                float dv = 0.f;
                if (s_bs[tid] >= 0) {
                    dv = s_rowdot[tid];
                    const int rb = s_bs[tid] - w0;  // first row of this row's block
                    const int E = s_exp[tid] + s_pref[rb];
                    k = 14 - a.prescale_c - E;
                    k = k < -60 ? -60 : (k > 60 ? 60 : k);
                    if (!s_rownz[tid]) k = 0;
                }
                a.delta[(size_t)h * T + t] = dv;
                a.prescale[(size_t)h * T + t] = (int8_t)k;
            }
        }
    }
}

}  // namespace

hipError_t launch_quant(const QuantArgs& a, int D, bool prep, hipStream_t stream)
{
    const dim3 grid((a.T + 31) / 32, a.H);
    if (a.T == 0) return hipSuccess;
    if (D == 128) {
        if (prep) hipLaunchKernelGGL((quant_kernel<128, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((quant_kernel<128, false>), grid, dim3(256), 0, stream, a);
    } else {
        if (prep) hipLaunchKernelGGL((quant_kernel<64, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((quant_kernel<64, false>), grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace flamia
