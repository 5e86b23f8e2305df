"""Small problem builders shared by the oracle pin tests (CPU only)."""
import numpy as np

import oracle
import workloads


def small_problem(seed, lens, Hq, Hkv, d, causal=True, capacity=None, scale_q=1.0, do_std=1.0):
    T = capacity if capacity is not None else int(sum(lens))
    w = workloads.make("small", seed, T, lens, Hq, Hkv, d,
                       flags=workloads.FLAG_CAUSAL if causal else 0, do_std=do_std)
    if scale_q != 1.0:
        q = workloads.bf16_bits_to_f32(w.q) * np.float32(scale_q)
        w.q = workloads.f32_to_bf16_bits(q)
    return w


def quantized_operands(w, block=32, rule=0):
    q = oracle.quantize(w.q, w.cu, block=block, rule=rule)
    k = oracle.quantize(w.k, w.cu, block=block, rule=rule)
    v = oracle.quantize(w.v, w.cu, block=block, rule=rule)
    return q, k, v


def mirror_pipeline(w, block=32, rule=0, per_row_ds=False, scale=None):
    """Quantize -> microscaled forward (bf16 O, f32 LSE as saved) -> backward
    prep -> dQ, dK, dV.  Returns a dict of every intermediate."""
    q, k, v = quantized_operands(w, block, rule)
    ops = oracle.Operands.from_codes(q, k, v)
    O64, LSE64 = oracle.attn_fwd(w.cu, ops, scale=scale, causal=w.causal)
    O = oracle.to_bf16(O64)
    LSE = LSE64.astype(np.float32)
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, O, k[1], v[1], w.Hkv, scale=scale,
                                      causal=w.causal, block=block)
    G = oracle.dequantize(gc, ge)
    lse = LSE.astype(np.float64)
    dQ = oracle.bwd_dq(w.cu, ops, G, D, lse, scale=scale, causal=w.causal, per_row_ds=per_row_ds)
    dK, dV = oracle.bwd_dkdv(w.cu, ops, G, D, lse, scale=scale, causal=w.causal,
                             per_row_ds=per_row_ds)
    return dict(q=q, k=k, v=v, ops=ops, O64=O64, O=O, LSE=LSE, gc=gc, ge=ge, G=G, D=D,
                kpre=kpre, dQ=dQ, dK=dK, dV=dV)
