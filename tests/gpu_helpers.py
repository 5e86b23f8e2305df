"""Helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded workloads and bring results back as numpy arrays."""
import sys

import numpy as np

import oracle
import workloads
from oracle import metrics


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


def run_gpu(w, flags=None, scale=0.0, backward=True, scale_mode=0):
    """Quantize, forward and (optionally) backward on the GPU."""
    import torch
    from bit_causal_flash_amd import flamia as F
    flags = (F.FLAMIA_CAUSAL if w.causal else 0) if flags is None else flags
    cu = dev(w.cu.astype(np.int32))
    p = F.make_problem(cu, w.T, w.Hq, w.Hkv, w.d, scale, flags)
    x = {n: dev(getattr(w, n).view(np.int16)) for n in ("q", "k", "v", "do")}
    q = F.quantize(p, x["q"], w.Hq, scale_mode)
    k = F.quantize(p, x["k"], w.Hkv, scale_mode)
    v = F.quantize(p, x["v"], w.Hkv, scale_mode)
    o, lse = F.attn_fwd(p, q, k, v)
    out = dict(qc=host(q[0]), qe=host(q[1]), kc=host(k[0]), ke=host(k[1]), vc=host(v[0]),
               ve=host(v[1]), O=host(o).view(np.uint16), LSE=host(lse))
    if backward:
        dq, dk, dv, ws = F.attn_bwd(p, q, k, v, o, lse, x["do"].view(torch.bfloat16))
        torch.cuda.synchronize()
        L = F.flamia_attn_bwd_workspace_layout(p)
        wsn = host(ws)
        T, Hq, d = w.T, w.Hq, w.d
        out.update(
            dQ=host(dq).view(np.uint16), dK=host(dk).view(np.uint16), dV=host(dv).view(np.uint16),
            gc=wsn[L.do_codes:L.do_codes + T * Hq * d].reshape(T, Hq, d),
            ge=wsn[L.do_exps:L.do_exps + Hq * T].reshape(Hq, T),
            D=wsn[L.delta:L.delta + 4 * Hq * T].view(np.float32).reshape(Hq, T),
            kpre=wsn[L.dq_prescale:L.dq_prescale + Hq * T].view(np.int8).reshape(Hq, T))
    torch.cuda.synchronize()
    return out


def run_gpu_exact(w):
    """The exact-scale path on the GPU: per-token quantizer, the E2M1 views of
    Q and K when the workload asks for the score view, forward, backward."""
    import torch
    from bit_causal_flash_amd import flamia as F
    fp4 = bool(w.flags & workloads.FLAG_FP4_SCORE)
    flags = F.FLAMIA_CAUSAL | F.FLAMIA_EXACT | (F.FLAMIA_FP4_SCORE if fp4 else 0)
    p = F.make_problem(dev(w.cu.astype(np.int32)), w.T, w.Hq, w.Hkv, w.d, 0.0, flags)
    x = {n: dev(getattr(w, n).view(np.int16)) for n in ("q", "k", "v", "do")}
    q = F.quantize(p, x["q"], w.Hq, F.FLAMIA_SCALE_PER_TOKEN)
    k = F.quantize(p, x["k"], w.Hkv, F.FLAMIA_SCALE_PER_TOKEN)
    v = F.quantize(p, x["v"], w.Hkv, F.FLAMIA_SCALE_PER_TOKEN)
    f4 = (F.quantize_nvfp4(p, x["q"], w.Hq), F.quantize_nvfp4(p, x["k"], w.Hkv)) if fp4 else None
    o, lse = F.attn_fwd(p, q, k, v, fp4=f4)
    dq, dk, dv, ws = F.attn_bwd(p, q, k, v, o, lse, x["do"].view(torch.bfloat16), fp4=f4)
    torch.cuda.synchronize()
    L = F.flamia_attn_bwd_workspace_layout(p)
    wsn = host(ws)
    T, Hq, d = w.T, w.Hq, w.d
    out = dict(qc=host(q[0]), qe=host(q[1]), kc=host(k[0]), ke=host(k[1]), vc=host(v[0]),
               ve=host(v[1]), O=host(o).view(np.uint16), LSE=host(lse),
               dQ=host(dq).view(np.uint16), dK=host(dk).view(np.uint16),
               dV=host(dv).view(np.uint16),
               gc=wsn[L.do_codes:L.do_codes + T * Hq * d].reshape(T, Hq, d),
               ge=wsn[L.do_exps:L.do_exps + Hq * T].reshape(Hq, T),
               D=wsn[L.delta:L.delta + 4 * Hq * T].view(np.float32).reshape(Hq, T),
               kpre=wsn[L.dq_prescale:L.dq_prescale + Hq * T].view(np.int8).reshape(Hq, T))
    if fp4:
        out.update(q4=host(f4[0][0]), q4s=host(f4[0][1]), k4=host(f4[1][0]), k4s=host(f4[1][1]))
    return out


def oracle_operands(w, block=32):
    q = oracle.quantize(w.q, w.cu, block=block)
    k = oracle.quantize(w.k, w.cu, block=block)
    v = oracle.quantize(w.v, w.cu, block=block)
    return q, k, v


def check_fwd(got_O, got_LSE, ref_O64, ref_LSE, ties=None, tag=""):
    """Forward parity on matching row sets.  O: bf16 bits [n][d] vs FP64 [n][d];
    LSE: [n] f32 vs FP64; ties: [n][2] the oracle's rounding-tie bounds
    (|dO| and relative |dl| that flips of near-tie weights could cause).
    Tolerances: O cosine >= 0.9995; every row within 1e-2 max|O| plus its tie
    bound; LSE within 1e-5 (1 + |LSE|) plus -ln(1 - tie_l), the larger of the
    moves of ln l when l changes by a relative tie_l up (ln(1 + tie_l)) or
    down (-ln(1 - tie_l)).  The GPU scores in
    FP32 and the oracle in FP64, so a weight within FP32 noise of an E4M3
    rounding midpoint may round either way; rows that need that allowance are
    counted and reported."""
    Og = oracle.bf16_to_float(got_O).reshape(-1, np.shape(got_O)[-1])
    Or = oracle.bf16_to_float(oracle.to_bf16(ref_O64)).reshape(Og.shape)
    tie = np.zeros((Og.shape[0], 2)) if ties is None else np.asarray(ties).reshape(-1, 2)
    rep = metrics.report(Og, Or)
    row_abs = np.abs(Og - Or).max(axis=1) if Og.size else np.zeros(0)
    base = 1e-2 * rep["max_ref"]
    needs_tie = row_abs > base
    log("%s O: %s rows beyond 1e-2 max|O| %d/%d, all within their tie bound: %s" %
        (tag, rep, int(needs_tie.sum()), row_abs.size, bool(np.all(row_abs <= base + tie[:, 0]))))
    assert rep["cos"] >= 0.9995, rep
    badr = np.nonzero(row_abs > base + tie[:, 0])[0]
    for i in badr[:5]:
        log("  O row %d: |d| %.4g base %.4g tie %.4g" % (i, row_abs[i], base, tie[i, 0]))
    assert badr.size == 0, "O rows beyond tolerance + tie bound"
    assert needs_tie.sum() <= max(2, 0.05 * row_abs.size)
    lg = np.asarray(got_LSE, dtype=np.float64).ravel()
    lr = np.asarray(ref_LSE, dtype=np.float64).ravel()
    fin = np.isfinite(lr)
    assert np.array_equal(np.isfinite(lg), fin)
    dl = np.where(fin, np.abs(lg - np.where(fin, lr, 0.0)), 0.0)
    allow = 1e-5 * (1.0 + np.abs(np.where(fin, lr, 0.0))) - np.log1p(-np.minimum(tie[:, 1], 1.0 - 1e-12))
    if fin.any():
        log("%s LSE: max |d| %.3g, rows needing the tie allowance %d" %
            (tag, dl[fin].max(), int(np.sum(dl[fin] > 1e-5 * (1 + np.abs(lr[fin]))))))
    badl = np.nonzero(fin & (dl > allow))[0]
    for i in badl[:5]:
        log("  LSE row %d: |d| %.4g allow %.4g (LSE %.4g, tie_l %.3g)" %
            (i, dl[i], allow[i], lr[i], tie[i, 1]))
    assert badl.size == 0


def dq_tiles(cu, T, causal):
    """Number of 128-key tiles whose FP16 partials reach each row's dQ."""
    n = np.zeros(T, dtype=np.int64)
    for s, e in zip(cu[:-1], cu[1:]):
        s, e = int(s), int(e)
        pos = np.arange(e - s)
        n[s:e] = (pos // 128 + 1) if causal else ((e - s + 127) // 128)
    return n


def check_grad(got, ref64, tag, tie=None, rows=None, acc=None, ntiles=None, absm=None,
               cos_min=0.995, row_max=5e-2):
    """Gradient parity: cosine >= 0.995 and per-row max relative error <=
    5e-2 (relative to the row's largest entry, floored at 1e-3 of the largest
    entry overall), plus, per row, only what the arithmetic can explain:
      - tie: the oracle's bound on what flips of near-tie P^ / dS^ elements
        could move the row (FP32 vs FP64 evaluation), and
      - for dQ, the FP16 accumulation of the per-128-key-tile partials that
        the method prescribes: (n_tiles + 1) 2^-11 acc, acc being the sum
        over tiles of each tile partial's largest magnitude, plus two bf16
        roundings;
      - the FP8 matrix cores' own rounding of the gradient product: 2^-11 of
        the row's largest sum of absolute terms (absm).
    Rows that need an allowance are counted and reported.  `rows` restricts
    the check to a boolean [T][H] mask (sampled rows)."""
    g = oracle.bf16_to_float(got)
    r = oracle.bf16_to_float(oracle.to_bf16(ref64))
    pick = (lambda x: None if x is None else np.asarray(x)[rows]) if rows is not None else \
        (lambda x: x)
    g, r, tie, acc, ntiles, absm = (pick(g), pick(r), pick(tie), pick(acc), pick(ntiles),
                                    pick(absm))
    g = g.reshape(-1, g.shape[-1])
    r = r.reshape(-1, r.shape[-1])
    n = g.shape[0]
    tie = np.zeros(n) if tie is None else np.asarray(tie, dtype=np.float64).ravel()
    rep = metrics.report(g, r)
    diff = np.abs(g - r).max(axis=1)
    rmax = np.abs(r).max(axis=1)
    denom = np.maximum(rmax, 1e-3 * rep["max_ref"])
    base = row_max * denom
    accb = np.zeros(n)
    if acc is not None:
        accb = (np.asarray(ntiles).ravel() + 1) * 2.0 ** -11 * np.asarray(acc).ravel() + \
            2.0 ** -7 * rmax
    mfma = np.zeros(n) if absm is None else 2.0 ** -11 * np.asarray(absm).ravel()
    over = diff > base
    log("%s: %s rows beyond %.0e: %d/%d (within the tie bound %d, within the FP16 "
        "accumulation bound %d, within the MFMA rounding bound %d)" %
        (tag, rep, row_max, int(over.sum()), n, int(np.sum(over & (diff <= base + tie))),
         int(np.sum(over & (diff <= base + accb))), int(np.sum(over & (diff <= base + mfma)))))
    assert rep["cos"] >= cos_min, rep
    bad = diff > base + tie + accb + mfma
    for i in np.nonzero(bad)[0][:5]:
        log("  row %d: |d| %.4g base %.4g tie %.4g acc %.4g mfma %.4g rowmax %.4g" %
            (i, diff[i], base[i], tie[i], accb[i], mfma[i], rmax[i]))
    assert not np.any(bad), "rows beyond tolerance + bounds: %s" % np.nonzero(bad)[0][:10]
    return diff / denom
