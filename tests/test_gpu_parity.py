"""GPU parity: the HIP path through the C ABI against the FP64 oracle on the
same seeded inputs.  Codes, exponents and prescale exponents bit-exact;
forward and backward within the stated tolerances."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import Backward, check_fwd, dev, fwd_ties, host, log, oracle_operands, run_gpu

pytestmark = pytest.mark.gpu

SMALL = [
    # name, lens, capacity, Hq, Hkv, d, causal
    ("one_doc_d64", [256], 256, 1, 1, 64, True),
    ("ragged_d128", [300, 7, 129, 1, 64], 520, 2, 2, 128, True),
    ("gqa_d128", [190, 333], 560, 4, 2, 128, True),
    ("gqa_d64_tail", [45, 250, 97], 400, 6, 2, 64, True),
    ("noncausal_d128", [150, 80, 33], 300, 2, 1, 128, False),
    # empty documents at the start, in the middle and at the end, a 1-token
    # document and padding rows
    ("empty_docs_d64", [0, 50, 0, 0, 33, 1, 0], 100, 2, 1, 64, True),
    ("empty_docs_noncausal_d128", [0, 70, 0, 40, 0], 128, 2, 2, 128, False),
    # few, long backward tickets (8 q heads per kv head): the 256-key backward
    # splits the items of cost >= 8 query tiles (64 iterations) into two
    # halves whose dK / dV slots the pair kernel adds up -- the first key
    # tiles of the 700- and 520-token documents, every key tile of the
    # 600-token one
    ("split_gqa_d128", [700, 300, 520], 1536, 8, 1, 128, True),
    ("split_noncausal_d64", [600, 150], 760, 8, 1, 64, False),
]


def _workload(name, lens, cap, Hq, Hkv, d, causal, seed=0):
    return workloads.make(name, seed, cap, lens, Hq, Hkv, d,
                          flags=workloads.FLAG_CAUSAL if causal else 0)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_forward_backward(case):
    name, lens, cap, Hq, Hkv, d, causal = case
    log("case %s" % name)
    _check_case(_workload(*case), name)


@pytest.mark.parametrize("d", [64, 128])
def test_rising_scores_take_the_rescale_path(d):
    """Scores that climb by about 50 (base-2 logits) along each document: the
    forward keeps O and l in units of each query's first reference and moves
    that base (with a rescale) once the reference has risen more than 32 above
    it, which the later queries here do.  Parity as in the small cases."""
    lens, cap, Hq, Hkv = [256, 200], 480, 2, 1
    w = workloads.make("rising_d%d" % d, 7, cap, lens, Hq, Hkv, d)
    rng = np.random.default_rng(8)
    q = 1.0 + 0.05 * rng.standard_normal((cap, Hq, d))
    k = 0.05 * rng.standard_normal((cap, Hkv, d)) + 1.0
    alpha = np.zeros(cap)
    for s, e in zip(w.cu[:-1], w.cu[1:]):
        # q . k reaches d alpha: base-2 logits up to about 50
        alpha[s:e] = np.linspace(0.0, 50.0 / (d ** 0.5 * 1.4426950408889634), e - s)
    k *= alpha[:, None, None]
    w.q = workloads.f32_to_bf16_bits(q.astype(np.float32))
    w.k = workloads.f32_to_bf16_bits(k.astype(np.float32))
    # the last query of the first document: its integer reference (the ceiling
    # of its largest logit) rises by more than 32 after the first 64-key step
    s2 = (q[255, 0] @ k[:256, 0].T) / d ** 0.5 * 1.4426950408889634
    assert np.ceil(s2.max()) - np.ceil(s2[:64].max()) > 33
    _check_case(w, "rising_d%d" % d)


def _check_case(w, name):
    Hq, Hkv, d, causal = w.Hq, w.Hkv, w.d, w.causal
    g = run_gpu(w)
    # quantizer: bit-exact
    q, k, v = oracle_operands(w)
    for tag, (c, e) in (("q", q), ("k", k), ("v", v)):
        assert np.array_equal(g[tag + "c"], c), tag + " codes"
        assert np.array_equal(g[tag + "e"], e), tag + " exps"
    # forward against the microscaled oracle
    ops = oracle.Operands.from_codes(q, k, v)
    O, L = oracle.attn_fwd(w.cu, ops, causal=causal, mode=oracle.MODE_TILED, kblock=64)
    ties = fwd_ties(w.cu, ops, causal=causal)
    check_fwd(g["O"].reshape(-1, d), g["LSE"].T.ravel(), O.reshape(-1, d), L.T.ravel(),
              ties.transpose(1, 0, 2).reshape(-1, 2), tag=name)
    # causal: the first token of every document sees only itself, so O equals
    # its dequantized V row exactly
    for s, e_ in zip(w.cu[:-1], w.cu[1:]):
        if e_ > s and causal:
            for h in range(Hq):
                assert np.array_equal(g["O"][s, h], oracle.to_bf16(ops.V[s, h * Hkv // Hq]))
    # backward, from the GPU's saved O and LSE
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, g["O"], k[1], v[1], Hkv, causal=causal)
    assert np.array_equal(g["gc"], gc) and np.array_equal(g["ge"], ge)
    assert np.array_equal(g["kpre"].astype(np.int32), kpre)
    assert np.allclose(g["D"], D, rtol=1e-4, atol=1e-6 * np.abs(D).max())
    G = oracle.dequantize(gc, ge)
    lse = g["LSE"].astype(np.float64)
    Backward(w.cu, ops, G, D, lse, kpre=kpre, causal=causal).check(g, name)
    # padding rows
    n = int(w.cu[-1])
    assert np.all(g["O"][n:] == 0) and np.all(np.isinf(g["LSE"][:, n:]))
    assert np.all(g["dQ"][n:] == 0) and np.all(g["dK"][n:] == 0) and np.all(g["dV"][n:] == 0)


def test_quantizer_per_token_mode_bit_exact():
    w = _workload("pt", [100, 61], 170, 3, 1, 128, True)
    g = run_gpu(w, backward=False, scale_mode=1)
    c, e = oracle.quantize(w.q, w.cu, block=1)
    assert np.array_equal(g["qc"], c) and np.array_equal(g["qe"], e)


def test_quantizer_edge_values_bit_exact():
    # zero blocks, a huge outlier, bf16 subnormals and negative zeros
    rng = np.random.default_rng(3)
    x = rng.standard_normal((96, 2, 64)).astype(np.float32)
    x[0:32] = 0.0
    x[40, 1, 5] = 3.0e38
    x[70:80] *= np.float32(1e-39)
    x[81, 0, :] = -0.0
    w = workloads.make("edge", 0, 96, [37, 59], 2, 2, 64)
    w.q = workloads.f32_to_bf16_bits(x)
    g = run_gpu(w, backward=False)
    c, e = oracle.quantize(w.q, w.cu)
    assert np.array_equal(g["qc"], c) and np.array_equal(g["qe"], e)


@pytest.mark.gpu
def test_quantizer_nvfp4_bit_exact():
    """E2M1 score view (E4M3 scale per 16 features): random groups, zero
    groups, a group past the scale's range, bf16 subnormals, values on the
    lattice midpoints (ties to the even code) and padding rows."""
    from bit_causal_flash_amd import flamia as F
    rng = np.random.default_rng(11)
    T, H, d = 80, 3, 64
    x = rng.standard_normal((T, H, d)).astype(np.float32)
    x[0:4] = 0.0
    x[5, 1, 3] = 3.0e38
    x[6:9] *= np.float32(1e-39)
    x[9, 0, :16] = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                             -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 0.0], np.float32)
    x[10, 2, 16:32] = np.linspace(-7.0, 7.0, 16).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    cu = np.array([0, 30, 71], np.int32)  # rows 71.. are padding
    log("case nvfp4 T=%d H=%d d=%d" % (T, H, d))
    p = F.make_problem(dev(cu), T, H, H, d, 0.0, F.FLAMIA_CAUSAL)
    codes, scales = F.quantize_nvfp4(p, dev(bits.view(np.int16)), H)
    rc, rs = oracle.quantize_nvfp4(bits, cu)
    assert np.array_equal(host(codes), rc), "codes"
    assert np.array_equal(host(scales), rs), "scales"


def _exact_case(name, lens, cap, Hq, Hkv, d, fp4, seed=5):
    """Per-token operands (and the E2M1 score views) on the GPU and in the
    oracle, for the exact-scale option."""
    import torch
    from bit_causal_flash_amd import flamia as F
    w = workloads.make(name, seed, cap, lens, Hq, Hkv, d)
    flags = F.FLAMIA_CAUSAL | F.FLAMIA_EXACT | (F.FLAMIA_FP4_SCORE if fp4 else 0)
    p = F.make_problem(dev(w.cu.astype(np.int32)), w.T, Hq, Hkv, d, 0.0, flags)
    x = {n: dev(getattr(w, n).view(np.int16)) for n in ("q", "k", "v", "do")}
    q = F.quantize(p, x["q"], Hq, F.FLAMIA_SCALE_PER_TOKEN)
    k = F.quantize(p, x["k"], Hkv, F.FLAMIA_SCALE_PER_TOKEN)
    v = F.quantize(p, x["v"], Hkv, F.FLAMIA_SCALE_PER_TOKEN)
    f4 = (F.quantize_nvfp4(p, x["q"], Hq), F.quantize_nvfp4(p, x["k"], Hkv)) if fp4 else None
    o, lse = F.attn_fwd(p, q, k, v, fp4=f4)
    torch.cuda.synchronize()
    rq, rk, rv = (oracle.quantize(getattr(w, n), w.cu, block=1) for n in ("q", "k", "v"))
    for tag, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert np.array_equal(host(got[0]), ref[0]) and np.array_equal(host(got[1]), ref[1]), tag
    r4 = None
    if fp4:
        r4 = (oracle.quantize_nvfp4(w.q, w.cu), oracle.quantize_nvfp4(w.k, w.cu))
        for (gc, gs), (rc, rs) in zip(f4, r4):
            assert np.array_equal(host(gc), rc) and np.array_equal(host(gs), rs)
    ops = oracle.Operands.from_codes(rq, rk, rv, *(r4 or (None, None)))
    return w, p, (q, k, v, f4, x), (o, lse), ops


@pytest.mark.parametrize("fp4", [False, True], ids=["exact", "exact_fp4"])
@pytest.mark.parametrize("d", [64, 128])
def test_exact_forward(fp4, d):
    log("case exact forward fp4=%s d=%d" % (fp4, d))
    w, p, _, (o, lse), ops = _exact_case("exact", [160, 97], 270, 4, 2, d, fp4)
    O, L = oracle.attn_fwd(w.cu, ops, causal=True, mode=oracle.MODE_TILED, kblock=64)
    ties = fwd_ties(w.cu, ops)
    check_fwd(host(o).view(np.uint16).reshape(-1, d), host(lse).T.ravel(), O.reshape(-1, d),
              L.T.ravel(), ties.transpose(1, 0, 2).reshape(-1, 2), tag="exact fp4=%s d=%d" % (fp4, d))


EXACT_BWD = [(64, False), (64, True), (128, False)]


@pytest.mark.parametrize("d,fp4", EXACT_BWD, ids=["exact_d64", "exact_fp4_d64", "exact_d128"])
def test_exact_backward(d, fp4, lens=(230, 97, 40), cap=400, Hq=4, Hkv=2):
    """Exact-scale backward: per-token dO, folded exponents and per-(query
    row, 32-key block) dS exponents for dQ, against the oracle's per-row dS
    backward on the same per-token operands."""
    import torch
    from bit_causal_flash_amd import flamia as F
    log("case exact backward fp4=%s d=%d Hq=%d Hkv=%d" % (fp4, d, Hq, Hkv))
    w, p, (q, k, v, f4, x), (o, lse), ops = _exact_case("exact_bwd", list(lens), cap, Hq, Hkv,
                                                        d, fp4, seed=9)
    dq, dk, dv, ws = F.attn_bwd(p, q, k, v, o, lse, x["do"].view(torch.bfloat16), fp4=f4)
    torch.cuda.synchronize()
    T = w.T
    L = F.flamia_attn_bwd_workspace_layout(p)
    wsn = host(ws)
    O = host(o).view(np.uint16)
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, O, host(k[1]), host(v[1]), Hkv, block=1)
    assert np.array_equal(wsn[L.do_codes:L.do_codes + T * Hq * d].reshape(T, Hq, d), gc)
    assert np.array_equal(wsn[L.do_exps:L.do_exps + Hq * T].reshape(Hq, T), ge)
    assert np.array_equal(wsn[L.dq_prescale:L.dq_prescale + Hq * T].view(np.int8).reshape(Hq, T)
                          .astype(np.int32), kpre)
    G = oracle.dequantize(gc, ge)
    lse64 = host(lse).astype(np.float64)
    tag = "exact fp4=%s d=%d" % (fp4, d)
    Backward(w.cu, ops, G, D, lse64, kpre=kpre, per_row_ds=True).check(
        dict(dQ=host(dq).view(np.uint16), dK=host(dk).view(np.uint16), dV=host(dv).view(np.uint16)),
        tag)
    n = int(w.cu[-1])
    for t in (dq, dk, dv):
        assert np.all(host(t)[n:] == 0)


def test_exact_backward_empty_documents():
    """The exact-scale path (E2M1 score view) with empty documents between and
    after the others."""
    test_exact_backward(64, True, lens=(0, 61, 0, 140, 0), cap=220)


def test_exact_backward_split_tickets():
    """The exact-scale path (E2M1 score view) with 8 q heads per kv head, so
    that the backward splits its longest tickets and the pair kernel adds the
    halves' dK / dV."""
    test_exact_backward(64, True, lens=(700, 300, 520), cap=1536, Hq=8, Hkv=1)


@pytest.mark.parametrize("mode", ["tokblock", "per_token", "rotated"])
def test_fused_qkv_quantizer_bit_exact(mode):
    """Q, K, V in one launch: the same codes and exponents as the oracle (and
    so as three separate calls), with GQA head counts and padding rows."""
    import torch
    from bit_causal_flash_amd import flamia as F
    log("case fused qkv quantizer %s" % mode)
    w = workloads.make("qkv", 3, 420, [150, 7, 200, 0, 33], 6, 2, 128)
    scale_mode = {"tokblock": F.FLAMIA_SCALE_TOKBLOCK32, "per_token": F.FLAMIA_SCALE_PER_TOKEN,
                  "rotated": F.FLAMIA_SCALE_TOKBLOCK32 | F.FLAMIA_SCALE_ROTATE}[mode]
    p = F.make_problem(dev(w.cu.astype(np.int32)), w.T, w.Hq, w.Hkv, w.d, 0.0, F.FLAMIA_CAUSAL)
    x = [dev(getattr(w, n).view(np.int16)) for n in ("q", "k", "v")]
    got = F.quantize_qkv(p, *x, scale_mode=scale_mode)
    torch.cuda.synchronize()
    blk = 1 if mode == "per_token" else 32
    for i, n in enumerate(("q", "k", "v")):
        if mode == "rotated" and n != "v":
            rc, re = oracle.quantize_rotated(getattr(w, n), w.cu, block=blk)
        else:
            rc, re = oracle.quantize(getattr(w, n), w.cu, block=blk)
        assert np.array_equal(host(got[i][0]), rc), n + " codes"
        assert np.array_equal(host(got[i][1]), re), n + " exponents"


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_all_documents_empty(causal):
    """Every row is padding: three zero-length documents over 64 rows of
    random data.  Codes 0 and exponent bytes 127 (as the oracle's quantizer
    gives), O = 0, LSE = +inf, the backward preparation's outputs as the
    oracle's, and zero gradients."""
    w = workloads.make("all_empty", 0, 64, [0, 0, 0], 2, 1, 64,
                       flags=workloads.FLAG_CAUSAL if causal else 0)
    log("all documents empty, causal=%d" % causal)
    g = run_gpu(w)
    q, k, v = oracle_operands(w)
    for tag, (c, e) in (("q", q), ("k", k), ("v", v)):
        assert np.all(c == 0) and np.all(e == 127)
        assert np.array_equal(g[tag + "c"], c), tag + " codes"
        assert np.array_equal(g[tag + "e"], e), tag + " exps"
    assert np.all(g["O"] == 0)
    assert np.all(np.isinf(g["LSE"])) and np.all(g["LSE"] > 0)
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, g["O"], k[1], v[1], w.Hkv, causal=causal)
    assert np.array_equal(g["gc"], gc) and np.array_equal(g["ge"], ge)
    assert np.array_equal(g["kpre"].astype(np.int32), kpre)
    assert np.array_equal(g["D"], D.astype(np.float32))
    for t in ("dQ", "dK", "dV"):
        assert np.all(g[t] == 0), t
