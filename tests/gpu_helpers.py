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


# Evaluation error of the GPU's dot products of E4M3 codes, as a fraction of
# the sum of the absolute values of their terms: gfx950's FP8 matrix cores
# keep about 12 bits below the largest product inside one instruction
# (deviations from FP64 measured up to 2^-12.6 of that sum on random data),
# and FP32 VALU work adds far less; 2^-12 leaves a factor 1.5.  It decides
# which P^ / dS^ elements lie close enough to an E4M3 rounding midpoint that
# either rounding is a correct result; it never widens a tolerance by itself.
NOISE = 2.0 ** -12


def fwd_ties(cu, ops, rows=None, **kw):
    """The oracle's per-row tie bounds of the forward at NOISE, [Hq][T][2]."""
    return oracle.fwd_ties(cu, ops, NOISE, mode=oracle.MODE_TILED, kblock=64, rows=rows, **kw)


def check_fwd(got_O, got_LSE, ref_O64, ref_LSE, ties=None, tag=""):
    """Forward parity on matching row sets.  O: bf16 bits [n][d] vs FP64 [n][d];
    LSE: [n] f32 vs FP64; ties: [n][2] the oracle's rounding-tie bounds
    (|dO| and relative |dl| that flips of near-tie weights could cause).
    Tolerances: O cosine >= 0.9995; every row within 1e-2 max|O| plus its tie
    bound, and at most 5 % of the rows (or 2) needing the tie bound; LSE within
    1e-5 (1 + |LSE|) plus -ln(1 - tie_l), the larger of the moves of ln l when
    l changes by a relative tie_l up (ln(1 + tie_l)) or down (-ln(1 - tie_l)).
    The reference is the oracle's tile loop at the kernel's 64-key step (the
    weights are rounded against the running reference of each step)."""
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


def _closest_alternative(target, C, lo, hi):
    """Smallest max-abs residual target - x C found over lo <= x <= hi (a
    bounded least-squares solution: enough to show that a valid alternative
    exists, which is all the check needs)."""
    from scipy.optimize import lsq_linear
    if len(C) == 0:
        return float(np.abs(target).max())
    C = np.asarray(C, dtype=np.float64)
    lo, hi = np.asarray(lo, dtype=np.float64), np.asarray(hi, dtype=np.float64)
    x = lsq_linear(C.T, target, bounds=(lo, hi), method="bvls").x
    return float(np.abs(target - x @ C).max())


def check_grad(got, ref64, tag, alternatives=None, cos_min=0.995, row_max=5e-2, alt_max=1e-2,
               max_alt_frac=0.05):
    """Gradient parity on matching row sets: got bf16 bits (or float64
    values) [n][d], ref64 float64 [n][d].  Every row must have max relative
    error <= 5e-2 (relative to the row's largest reference entry, floored at
    1e-3 of the largest entry overall), cosine >= 0.995 overall.

    Several results are correct where an element of P^ or dS^ lies within the
    GPU's evaluation error (NOISE) of an E4M3 rounding midpoint: the method
    then allows either rounding (and the 32x32 block exponent can move when
    the block maximum sits at a threshold).  A row beyond 5e-2 passes only if
    such an alternative result explains it to within 1e-2 (alt_max, stricter
    than the tolerance itself, so that the freedom of many near-midpoint
    elements cannot absorb a real error): alternatives(k) returns
    (C [m][d], lo [m], hi [m]) for row k, the valid results being ref + x C
    with lo <= x <= hi.  At most 5 % of the rows (or 2) may need one.
    Returns a dict of the row statistics, which is also logged."""
    got = np.asarray(got)
    g = oracle.bf16_to_float(got) if got.dtype == np.uint16 else got.astype(np.float64)
    r = oracle.bf16_to_float(oracle.to_bf16(ref64))
    d = g.shape[-1]
    g, r = g.reshape(-1, d), r.reshape(-1, d)
    n = g.shape[0]
    rep = metrics.report(g, r)
    diff = np.abs(g - r).max(axis=1)
    rmax = np.abs(r).max(axis=1)
    denom = np.maximum(rmax, 1e-3 * rep["max_ref"])
    err = diff / denom
    over = np.nonzero(err > row_max)[0]
    resolved, worst_alt, failed = 0, 0.0, []
    for k in over:
        if alternatives is None:
            failed.append(k)
            continue
        C, lo, hi = alternatives(int(k))
        res = _closest_alternative(g[k] - r[k], C, lo, hi) / denom[k]
        worst_alt = max(worst_alt, res)
        if res <= alt_max:
            resolved += 1
        else:
            failed.append(k)
    stats = dict(rows=n, p50=float(np.median(err)) if n else 0.0,
                 p99=float(np.quantile(err, 0.99)) if n else 0.0,
                 max=float(err.max()) if n else 0.0, beyond=int(over.size),
                 resolved_by_alternative=resolved, worst_alternative_residual=worst_alt,
                 cos=rep["cos"])
    log("%s: %s per-row rel err p50 %.3g p99 %.3g max %.3g; rows beyond %.0e: %d/%d, "
        "within %.0e of an alternative rounding: %d (worst residual %.3g)" %
        (tag, rep, stats["p50"], stats["p99"], stats["max"], row_max, over.size, n, alt_max,
         resolved, worst_alt))
    for k in failed[:5]:
        log("  row %d: rel err %.4g |d| %.4g rowmax %.4g" % (k, err[k], diff[k], rmax[k]))
    assert rep["cos"] >= cos_min, rep
    assert not failed, "rows beyond tolerance with no valid alternative: %s" % failed[:10]
    assert over.size <= max(2, max_alt_frac * n), "too many rows needing an alternative"
    return stats


class Backward:
    """References and alternatives for the gradient checks of one problem:
    the oracle's microscaled backward on the GPU's own saved O / LSE (via D
    and LSE), dQ through the method's FP16 accumulation (the GPU's prescale
    exponents), dK and dV in FP64."""

    def __init__(self, cu, ops, G, D, lse, kpre=None, scale=None, causal=True, per_row_ds=False,
                 dq_tile=None):
        self.cu, self.ops, self.G = np.asarray(cu, np.int32), ops, np.ascontiguousarray(G)
        self.D = np.ascontiguousarray(D, dtype=np.float64)
        self.lse = np.ascontiguousarray(lse, dtype=np.float64)
        self.kpre = kpre
        self.scale = oracle.default_scale(ops.d) if scale is None else scale
        self.causal, self.per_row_ds = causal, per_row_ds
        # the key tile of the kernel's FP16 dQ partials: 256, except 128 with
        # per-token operands at d = 128
        self.dq_tile = dq_tile if dq_tile is not None else (128 if per_row_ds and ops.d == 128 else 256)
        self.kw = dict(scale=self.scale, causal=causal, per_row_ds=per_row_ds)
        self._ranges = {}

    def _block_start(self, t):
        b = int(np.searchsorted(self.cu, t, side="right") - 1)
        while self.cu[b + 1] <= t:
            b += 1
        return int(self.cu[b]) + 32 * ((int(t) - int(self.cu[b])) // 32)

    def dq(self, qblocks=None):
        """dQ reference over the listed (q head, block start) pairs: the FP16
        model when prescale exponents are given, else FP64."""
        if self.kpre is None:
            return oracle.bwd_dq(self.cu, self.ops, self.G, self.D, self.lse, qblocks=qblocks,
                                 **self.kw)
        return oracle.bwd_dq(self.cu, self.ops, self.G, self.D, self.lse, qblocks=qblocks,
                             kpre=np.asarray(self.kpre, np.int32), dq_tile=self.dq_tile,
                             **self.kw)[1]

    def dkdv(self, kblocks=None):
        return oracle.bwd_dkdv(self.cu, self.ops, self.G, self.D, self.lse, kblocks=kblocks,
                               **self.kw)

    def dq_alternatives(self, rows_th):
        """alternatives() for dQ rows listed as (token, q head) in check order."""
        ops, Hq, Hkv = self.ops, self.ops.Hq, self.ops.Hkv

        def alt(k):
            t, h = (int(x) for x in rows_th[k])
            q0 = self._block_start(t)
            key = ("q", h, q0)
            if key not in self._ranges:
                self._ranges[key] = oracle.dq_ranges(self.cu, ops, self.G, self.D, self.lse, h,
                                                     q0, NOISE, **self.kw)
            i, j, lo, hi = self._ranges[key]
            sel = i == t
            C = self.scale * ops.K[j[sel], h * Hkv // Hq]
            return C, lo[sel], hi[sel]
        return alt

    def dkdv_alternatives(self, rows_tg, which):
        """alternatives() for dV (which 0) or dK (which 1) rows listed as
        (token, kv head)."""
        ops = self.ops

        def alt(k):
            t, g = (int(x) for x in rows_tg[k])
            k0 = self._block_start(t)
            key = ("k", which, g, k0)
            if key not in self._ranges:
                self._ranges[key] = oracle.dkdv_ranges(self.cu, ops, self.G, self.D, self.lse, g,
                                                       k0, which, NOISE, **self.kw)
            h, i, j, lo, hi = self._ranges[key]
            sel = j == t
            C = self.G[i[sel], h[sel]] if which == 0 else self.scale * ops.Q[i[sel], h[sel]]
            return C, lo[sel], hi[sel]
        return alt

    def check(self, got, tag, qmask=None, kmask=None, frame=None):
        """Checks got = dict(dQ=..., dK=..., dV=...) (full [T][H][d] arrays of
        bf16 bits) on the rows of qmask [T][Hq] / kmask [T][Hkv] (None: all
        document rows).  frame maps a float64 gradient array to the frame the
        oracle computes in (the rotated one for the Hadamard option)."""
        T = self.ops.T
        n = int(self.cu[-1])
        if qmask is None:
            qmask = np.zeros((T, self.ops.Hq), bool)
            qmask[:n] = True
        if kmask is None:
            kmask = np.zeros((T, self.ops.Hkv), bool)
            kmask[:n] = True
        qb = sorted({(int(h), self._block_start(t)) for t, h in np.argwhere(qmask)})
        kb = sorted({(int(g), self._block_start(t)) for t, g in np.argwhere(kmask)})
        out = {}
        fr = (lambda x: x) if frame is None else frame

        def val(x):
            return fr(oracle.bf16_to_float(x))
        if "dQ" in got and qb:
            ref = self.dq(np.array(qb, np.int32))
            rows = np.argwhere(qmask)
            out["dQ"] = check_grad(val(got["dQ"])[qmask], ref[qmask], tag + " dQ",
                                   self.dq_alternatives(rows))
        if kb and ("dK" in got or "dV" in got):
            dK, dV = self.dkdv(np.array(kb, np.int32))
            rows = np.argwhere(kmask)
            if "dK" in got:
                out["dK"] = check_grad(val(got["dK"])[kmask], dK[kmask], tag + " dK",
                                       self.dkdv_alternatives(rows, 1))
            if "dV" in got:
                out["dV"] = check_grad(oracle.bf16_to_float(got["dV"])[kmask], dV[kmask],
                                       tag + " dV", self.dkdv_alternatives(rows, 0))
        return out
