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
