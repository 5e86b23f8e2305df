"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  Codes, exponents, dO codes and prescale exponents are
compared in full (bit-exact); forward rows and backward blocks are sampled
(document starts and ends, 32-token block boundaries and random interior
positions) and compared with the oracle element by element."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import (Backward, check_fwd, fwd_ties, log, oracle_operands, run_gpu,
                               run_gpu_exact)

pytestmark = pytest.mark.gpu


def _sample_tokens(cu, rng, per_doc=6, max_docs=None):
    """Sampled query tokens: each document's start, its first block
    boundary and end, and random interior positions; with max_docs, only the
    first document and max_docs - 1 others drawn at random."""
    docs = list(range(len(cu) - 1))
    if max_docs is not None and len(docs) > max_docs:
        docs = [0] + sorted(rng.choice(docs[1:], max_docs - 1, replace=False).tolist())
    toks = []
    for b in docs:
        s, e = int(cu[b]), int(cu[b + 1])
        if e <= s:
            continue
        toks += [s, min(s + 1, e - 1), min(s + 31, e - 1), min(s + 32, e - 1), e - 1]
        toks += list(rng.integers(s, e, size=per_doc))
    return sorted(set(toks))


def _masks(w, qstarts, heads, nk=12, max_kheads=4):
    """Rows of the sampled 32-query blocks (all heads listed) and of every
    nk-th of those blocks' starts as key blocks (their kv heads)."""
    qmask = np.zeros((w.T, w.Hq), dtype=bool)
    for h in heads:
        for t0 in qstarts:
            b = int(np.searchsorted(w.cu, t0, side="right") - 1)
            qmask[t0:min(t0 + 32, int(w.cu[b + 1])), h] = True
    kheads = sorted(set(h * w.Hkv // w.Hq for h in heads))[:max_kheads]
    kmask = np.zeros((w.T, w.Hkv), dtype=bool)
    for hk in kheads:
        for t0 in qstarts[:: max(1, len(qstarts) // nk)]:
            b = int(np.searchsorted(w.cu, t0, side="right") - 1)
            kmask[t0:min(t0 + 32, int(w.cu[b + 1])), hk] = True
    return qmask, kmask


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "packed_mha", "packed_gqa", "long_doc", "docs_16x4096",
                                  "docs_8192_224x256"])
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
    # the 8192 + 224 x 256 shape (most backward items a whole 256-token
    # document): the long document and 23 of the short ones
    toks = _sample_tokens(w.cu, rng, per_doc=8 if name != "long_doc" else 40,
                          max_docs=24 if name == "docs_8192_224x256" else None)
    heads = list(range(w.Hq)) if w.Hq <= 8 else list(rng.choice(w.Hq, 8, replace=False))
    rows = np.array([(h, t) for h in heads for t in toks], dtype=np.int32)
    ops = oracle.Operands.from_codes(q, k, v)
    O, L = oracle.attn_fwd(w.cu, ops, rows=rows, mode=oracle.MODE_TILED, kblock=64)
    ties = fwd_ties(w.cu, ops, rows=rows)
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
    qmask, kmask = _masks(w, oracle.doc_blocks(w.cu, toks), heads)
    Backward(w.cu, ops, G, D, lse, kpre=kpre).check(g, name, qmask=qmask, kmask=kmask)


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
    O, L = oracle.attn_fwd(w.cu, ops, rows=rows, mode=oracle.MODE_TILED, kblock=64)
    ties = fwd_ties(w.cu, ops, rows=rows)
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
    qmask, kmask = _masks(w, oracle.doc_blocks(w.cu, toks), heads)
    Backward(w.cu, ops, G, D, lse, kpre=kpre, per_row_ds=True).check(g, w.name, qmask=qmask,
                                                                      kmask=kmask)


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
    O, L = oracle.attn_fwd(w.cu, ops, scale=s, rows=rows, mode=oracle.MODE_TILED, kblock=64)
    ties = fwd_ties(w.cu, ops, scale=s, rows=rows)
    Og, Lg = host(o).view(np.uint16), host(lse)
    mask = np.zeros((T, Hq), dtype=bool)
    mask[rows[:, 1], rows[:, 0]] = True
    check_fwd(Og[mask], Lg.T[mask], O[mask], L.T[mask], ties.transpose(1, 0, 2)[mask], tag="hadamard")
    log("forward ok")
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, Og, rk[1], rv[1], Hkv, scale=s)
    G = oracle.dequantize(gc, ge)
    lse64 = Lg.astype(np.float64)
    qmask, kmask = _masks(w, oracle.doc_blocks(w.cu, toks), heads, nk=10, max_kheads=3)
    # compared in the rotated frame the oracle computes in: the GPU's dQ and
    # dK are dQ_r H and dK_r H with H H = d I, so dQ_r = dQ H / d
    Hm = oracle.hadamard_matrix(d)
    Backward(w.cu, ops, G, D, lse64, kpre=kpre, scale=s).check(
        dict(dQ=host(dq).view(np.uint16), dK=host(dk).view(np.uint16), dV=host(dv).view(np.uint16)),
        "hadamard", qmask=qmask, kmask=kmask, frame=lambda x: x @ Hm / d)


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
    O, L = oracle.attn_fwd(w.cu, ops, causal=False, rows=rows, mode=oracle.MODE_TILED, kblock=64)
    ties = fwd_ties(w.cu, ops, causal=False, rows=rows)
    mask = np.zeros((w.T, w.Hq), dtype=bool)
    mask[rows[:, 1], rows[:, 0]] = True
    check_fwd(g["O"][mask], g["LSE"].T[mask], O[mask], L.T[mask], ties.transpose(1, 0, 2)[mask],
              tag="non-causal")
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, g["O"], k[1], v[1], w.Hkv, causal=False)
    assert np.array_equal(g["gc"], gc) and np.array_equal(g["kpre"].astype(np.int32), kpre)
    G = oracle.dequantize(gc, ge)
    lse = g["LSE"].astype(np.float64)
    qmask, kmask = _masks(w, oracle.doc_blocks(w.cu, toks)[::2], heads, nk=4, max_kheads=3)
    Backward(w.cu, ops, G, D, lse, kpre=kpre, causal=False).check(g, "non-causal", qmask=qmask,
                                                                   kmask=kmask)
