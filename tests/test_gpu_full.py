"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  Codes, exponents, dO codes and prescale exponents are
compared in full (bit-exact); forward rows and backward blocks are sampled
(document starts and ends, 32-token block boundaries and random interior
positions) and compared with the oracle element by element."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import (check_fwd, check_grad, dq_tiles, log, oracle_operands, run_gpu,
                               run_gpu_exact)

pytestmark = pytest.mark.gpu


def _sample_tokens(cu, rng, per_doc=6):
    toks = []
    for s, e in zip(cu[:-1], cu[1:]):
        s, e = int(s), int(e)
        if e <= s:
            continue
        toks += [s, min(s + 1, e - 1), min(s + 31, e - 1), min(s + 32, e - 1), e - 1]
        toks += list(rng.integers(s, e, size=per_doc))
    return sorted(set(toks))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "packed_mha", "packed_gqa", "long_doc"])
def test_full_size_sampled(name):
    log("workload %s" % name)
    w = workloads.NAMED[name](0)
    g = run_gpu(w)
    log("gpu done")
    q, k, v = oracle_operands(w)
    for tag, (c, e) in (("q", q), ("k", k), ("v", v)):
        assert np.array_equal(g[tag + "c"], c), tag + " codes"
        assert np.array_equal(g[tag + "e"], e), tag + " exps"
    log("codes bit-exact")
    rng = np.random.default_rng(1)
    toks = _sample_tokens(w.cu, rng, per_doc=8 if name != "long_doc" else 40)
    heads = list(range(w.Hq)) if w.Hq <= 8 else list(rng.choice(w.Hq, 8, replace=False))
    rows = np.array([(h, t) for h in heads for t in toks], dtype=np.int32)
    ops = oracle.Operands.from_codes(q, k, v)
    O, L, ties = oracle.attn_fwd(w.cu, ops, rows=rows, mode=oracle.MODE_TILED, kblock=64,
                                   want_flags=True)
    mask = np.zeros((w.T, w.Hq), dtype=bool)
    mask[rows[:, 1], rows[:, 0]] = True
    check_fwd(g["O"][mask], g["LSE"].T[mask], O[mask], L.T[mask],
              ties.transpose(1, 0, 2)[mask], tag=name)
    log("forward ok")
    # backward preparation: bit-exact in full
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, g["O"], k[1], v[1], w.Hkv)
    assert np.array_equal(g["gc"], gc) and np.array_equal(g["ge"], ge)
    assert np.array_equal(g["kpre"].astype(np.int32), kpre)
    assert np.allclose(g["D"], D, rtol=1e-4, atol=1e-6 * np.abs(D).max())
    log("prep ok")
    G = oracle.dequantize(gc, ge)
    lse = g["LSE"].astype(np.float64)
    qstarts = oracle.doc_blocks(w.cu, toks)
    qblocks = np.array([(h, t0) for h in heads for t0 in qstarts], dtype=np.int32)
    dQ, tq, acc, aq = oracle.bwd_dq(w.cu, ops, G, D, lse, qblocks=qblocks, want_flags=True)
    nt = np.repeat(dq_tiles(w.cu, w.T, True)[:, None], w.Hq, axis=1)
    qmask = np.zeros((w.T, w.Hq), dtype=bool)
    for h, t0 in qblocks:
        b = int(np.searchsorted(w.cu, t0, side="right") - 1)
        qmask[t0:min(t0 + 32, int(w.cu[b + 1])), h] = True
    check_grad(g["dQ"], dQ, name + " dQ", tq, rows=qmask, acc=acc, ntiles=nt, absm=aq)
    kheads = sorted(set(h * w.Hkv // w.Hq for h in heads))[:4]
    kstarts = qstarts[:: max(1, len(qstarts) // 12)]
    kblocks = np.array([(hk, t0) for hk in kheads for t0 in kstarts], dtype=np.int32)
    dK, dV, tk, tv, ak, av = oracle.bwd_dkdv(w.cu, ops, G, D, lse, kblocks=kblocks, want_flags=True)
    kmask = np.zeros((w.T, w.Hkv), dtype=bool)
    for hk, t0 in kblocks:
        b = int(np.searchsorted(w.cu, t0, side="right") - 1)
        kmask[t0:min(t0 + 32, int(w.cu[b + 1])), hk] = True
    check_grad(g["dK"], dK, name + " dK", tk, rows=kmask, absm=ak)
    check_grad(g["dV"], dV, name + " dV", tv, rows=kmask, absm=av)


@pytest.mark.timeout(600)
def test_exact_option_full_size_sampled():
    """The exact-scale workload (8 documents x 2048, 16 / 4 heads, d = 64,
    per-token exponents, per-row dS exponents, E2M1 score view) at full size:
    codes, exponents, views, dO codes and prescale exponents in full; forward
    rows and backward blocks sampled against the oracle's exact-scale path."""
    w = workloads.NAMED["exact_option"](0)
    log("workload %s" % w.name)
    g = run_gpu_exact(w)
    log("gpu done")
    q, k, v = oracle_operands(w, block=1)
    for tag, (c, e) in (("q", q), ("k", k), ("v", v)):
        assert np.array_equal(g[tag + "c"], c), tag + " codes"
        assert np.array_equal(g[tag + "e"], e), tag + " exps"
    v4 = (oracle.quantize_nvfp4(w.q, w.cu), oracle.quantize_nvfp4(w.k, w.cu))
    for tag, (c, s) in (("q", v4[0]), ("k", v4[1])):
        assert np.array_equal(g[tag + "4"], c) and np.array_equal(g[tag + "4s"], s), tag + " view"
    log("codes and views bit-exact")
    rng = np.random.default_rng(2)
    toks = _sample_tokens(w.cu, rng, per_doc=8)
    heads = list(rng.choice(w.Hq, 6, replace=False))
    rows = np.array([(h, t) for h in heads for t in toks], dtype=np.int32)
    ops = oracle.Operands.from_codes(q, k, v, *v4)
    O, L, ties = oracle.attn_fwd(w.cu, ops, rows=rows, mode=oracle.MODE_TILED, kblock=64,
                                 want_flags=True)
    mask = np.zeros((w.T, w.Hq), dtype=bool)
    mask[rows[:, 1], rows[:, 0]] = True
    check_fwd(g["O"][mask], g["LSE"].T[mask], O[mask], L.T[mask],
              ties.transpose(1, 0, 2)[mask], tag=w.name)
    log("forward ok")
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, g["O"], k[1], v[1], w.Hkv, block=1)
    assert np.array_equal(g["gc"], gc) and np.array_equal(g["ge"], ge)
    assert np.array_equal(g["kpre"].astype(np.int32), kpre)
    assert np.allclose(g["D"], D, rtol=1e-4, atol=1e-6 * np.abs(D).max())
    log("prep ok")
    G = oracle.dequantize(gc, ge)
    lse = g["LSE"].astype(np.float64)
    qstarts = oracle.doc_blocks(w.cu, toks)
    qblocks = np.array([(h, t0) for h in heads for t0 in qstarts], dtype=np.int32)
    dQ, tq, acc, aq = oracle.bwd_dq(w.cu, ops, G, D, lse, per_row_ds=True, qblocks=qblocks,
                                    want_flags=True)
    nt = np.repeat(dq_tiles(w.cu, w.T, True)[:, None], w.Hq, axis=1)
    qmask = np.zeros((w.T, w.Hq), dtype=bool)
    for h, t0 in qblocks:
        qmask[t0:t0 + 32, h] = True
    check_grad(g["dQ"], dQ, w.name + " dQ", tq, rows=qmask, acc=acc, ntiles=nt, absm=aq)
    kheads = sorted(set(h * w.Hkv // w.Hq for h in heads))[:4]
    kstarts = qstarts[:: max(1, len(qstarts) // 12)]
    kblocks = np.array([(hk, t0) for hk in kheads for t0 in kstarts], dtype=np.int32)
    dK, dV, tk, tv, ak, av = oracle.bwd_dkdv(w.cu, ops, G, D, lse, per_row_ds=True,
                                             kblocks=kblocks, want_flags=True)
    kmask = np.zeros((w.T, w.Hkv), dtype=bool)
    for hk, t0 in kblocks:
        kmask[t0:t0 + 32, hk] = True
    check_grad(g["dK"], dK, w.name + " dK", tk, rows=kmask, absm=ak)
    check_grad(g["dV"], dV, w.name + " dV", tv, rows=kmask, absm=av)


@pytest.mark.timeout(600)
def test_hadamard_full_size_sampled():
    """The packed MHA workload with the Hadamard option at full size, in the
    benchmark's launch configuration: rotated codes and exponents in full,
    forward rows and backward blocks sampled against the oracle on the same
    rotated codes at scale / d, gradients rotated back."""
    import torch
    from bit_causal_flash_amd import flamia as F
    from tests.gpu_helpers import dev, host
    w = workloads.NAMED["packed_mha"](0)
    log("workload %s with the Hadamard rotation" % w.name)
    d, Hq, Hkv, T = w.d, w.Hq, w.Hkv, w.T
    p = F.make_problem(dev(w.cu.astype(np.int32)), T, Hq, Hkv, d, 0.0, F.FLAMIA_CAUSAL | F.FLAMIA_HADAMARD)
    x = {n: dev(getattr(w, n).view(np.int16)) for n in ("q", "k", "v", "do")}
    rot = F.FLAMIA_SCALE_TOKBLOCK32 | F.FLAMIA_SCALE_ROTATE
    q, k, v = F.quantize(p, x["q"], Hq, rot), F.quantize(p, x["k"], Hkv, rot), F.quantize(p, x["v"], Hkv)
    o, lse = F.attn_fwd(p, q, k, v)
    dq, dk, dv, ws = F.attn_bwd(p, q, k, v, o, lse, x["do"].view(torch.bfloat16))
    torch.cuda.synchronize()
    log("gpu done")
    rq, rk, rv = oracle.quantize_rotated(w.q, w.cu), oracle.quantize_rotated(w.k, w.cu), oracle.quantize(w.v, w.cu)
    for tag, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert np.array_equal(host(got[0]), ref[0]) and np.array_equal(host(got[1]), ref[1]), tag
    log("codes bit-exact")
    s = oracle.default_scale(d) / d
    ops = oracle.Operands.from_codes(rq, rk, rv)
    rng = np.random.default_rng(4)
    toks = _sample_tokens(w.cu, rng, per_doc=6)
    heads = list(rng.choice(Hq, 5, replace=False))
    rows = np.array([(h, t) for h in heads for t in toks], dtype=np.int32)
    O, L, ties = oracle.attn_fwd(w.cu, ops, scale=s, rows=rows, mode=oracle.MODE_TILED, kblock=64,
                                 want_flags=True)
    Og, Lg = host(o).view(np.uint16), host(lse)
    mask = np.zeros((T, Hq), dtype=bool)
    mask[rows[:, 1], rows[:, 0]] = True
    check_fwd(Og[mask], Lg.T[mask], O[mask], L.T[mask], ties.transpose(1, 0, 2)[mask], tag="hadamard")
    log("forward ok")
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, Og, rk[1], rv[1], Hkv, scale=s)
    G = oracle.dequantize(gc, ge)
    lse64 = Lg.astype(np.float64)
    qstarts = oracle.doc_blocks(w.cu, toks)
    qblocks = np.array([(h, t0) for h in heads for t0 in qstarts], dtype=np.int32)
    dQr, tq, acc, aq = oracle.bwd_dq(w.cu, ops, G, D, lse64, scale=s, qblocks=qblocks, want_flags=True)
    nt = np.repeat(dq_tiles(w.cu, T, True)[:, None], Hq, axis=1)
    qmask = np.zeros((T, Hq), dtype=bool)
    for h, t0 in qblocks:
        b = int(np.searchsorted(w.cu, t0, side="right") - 1)
        qmask[t0:min(t0 + 32, int(w.cu[b + 1])), h] = True
    # rows are rotated back whole, so the sampled blocks' rows are exact;
    # per-row allowances grow by at most d under the rotation
    check_grad(host(dq).view(np.uint16), oracle.unrotate(dQr), "hadamard dQ", d * tq, rows=qmask,
               acc=d * acc, ntiles=nt, absm=d * aq)
    kheads = sorted(set(h * Hkv // Hq for h in heads))[:3]
    kstarts = qstarts[:: max(1, len(qstarts) // 10)]
    kblocks = np.array([(hk, t0) for hk in kheads for t0 in kstarts], dtype=np.int32)
    dKr, dV, tk, tv, ak, av = oracle.bwd_dkdv(w.cu, ops, G, D, lse64, scale=s, kblocks=kblocks,
                                              want_flags=True)
    kmask = np.zeros((T, Hkv), dtype=bool)
    for hk, t0 in kblocks:
        b = int(np.searchsorted(w.cu, t0, side="right") - 1)
        kmask[t0:min(t0 + 32, int(w.cu[b + 1])), hk] = True
    check_grad(host(dk).view(np.uint16), oracle.unrotate(dKr), "hadamard dK", d * tk, rows=kmask,
               absm=d * ak)
    check_grad(host(dv).view(np.uint16), dV, "hadamard dV", tv, rows=kmask, absm=av)


@pytest.mark.timeout(600)
def test_noncausal_full_size_sampled():
    """The packed MHA workload without the causal mask (the non-causal
    variant of the same kernels), at full size: codes in full, forward rows
    and backward blocks sampled against the oracle."""
    w = workloads.NAMED["packed_mha"](0)
    w.flags &= ~workloads.FLAG_CAUSAL
    log("workload %s, non-causal" % w.name)
    g = run_gpu(w)
    q, k, v = oracle_operands(w)
    for tag, (c, e) in (("q", q), ("k", k), ("v", v)):
        assert np.array_equal(g[tag + "c"], c) and np.array_equal(g[tag + "e"], e), tag
    rng = np.random.default_rng(8)
    toks = _sample_tokens(w.cu, rng, per_doc=5)
    heads = list(rng.choice(w.Hq, 5, replace=False))
    rows = np.array([(h, t) for h in heads for t in toks], dtype=np.int32)
    ops = oracle.Operands.from_codes(q, k, v)
    O, L, ties = oracle.attn_fwd(w.cu, ops, causal=False, rows=rows, mode=oracle.MODE_TILED, kblock=64,
                                 want_flags=True)
    mask = np.zeros((w.T, w.Hq), dtype=bool)
    mask[rows[:, 1], rows[:, 0]] = True
    check_fwd(g["O"][mask], g["LSE"].T[mask], O[mask], L.T[mask], ties.transpose(1, 0, 2)[mask],
              tag="non-causal")
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, g["O"], k[1], v[1], w.Hkv, causal=False)
    assert np.array_equal(g["gc"], gc) and np.array_equal(g["kpre"].astype(np.int32), kpre)
    G = oracle.dequantize(gc, ge)
    lse = g["LSE"].astype(np.float64)
    qstarts = oracle.doc_blocks(w.cu, toks)
    qblocks = np.array([(h, t0) for h in heads for t0 in qstarts[::2]], dtype=np.int32)
    dQ, tq, acc, aq = oracle.bwd_dq(w.cu, ops, G, D, lse, causal=False, qblocks=qblocks, want_flags=True)
    nt = np.repeat(dq_tiles(w.cu, w.T, False)[:, None], w.Hq, axis=1)
    qmask = np.zeros((w.T, w.Hq), dtype=bool)
    for h, t0 in qblocks:
        b = int(np.searchsorted(w.cu, t0, side="right") - 1)
        qmask[t0:min(t0 + 32, int(w.cu[b + 1])), h] = True
    check_grad(g["dQ"], dQ, "non-causal dQ", tq, rows=qmask, acc=acc, ntiles=nt, absm=aq)
    kheads = sorted(set(h * w.Hkv // w.Hq for h in heads))[:3]
    kstarts = qstarts[:: max(1, len(qstarts) // 8)]
    kblocks = np.array([(hk, t0) for hk in kheads for t0 in kstarts], dtype=np.int32)
    dK, dV, tk, tv, ak, av = oracle.bwd_dkdv(w.cu, ops, G, D, lse, causal=False, kblocks=kblocks,
                                             want_flags=True)
    kmask = np.zeros((w.T, w.Hkv), dtype=bool)
    for hk, t0 in kblocks:
        b = int(np.searchsorted(w.cu, t0, side="right") - 1)
        kmask[t0:min(t0 + 32, int(w.cu[b + 1])), hk] = True
    check_grad(g["dK"], dK, "non-causal dK", tk, rows=kmask, absm=ak)
    check_grad(g["dV"], dV, "non-causal dV", tv, rows=kmask, absm=av)
