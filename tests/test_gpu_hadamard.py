"""GPU parity of the Hadamard option (FLAMIA review section 3 "Rotation,
range, and the alternative", Algorithm 1 step 02; jaehun.me section 3.4):
rotated-operand codes bit-exact against the oracle's FP32 fast transform, and
the forward / backward with rotated Q and K against the oracle on the same
rotated codes at softmax scale / d, with dQ and dK taken back by the oracle's
un-rotation."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import Backward, check_fwd, dev, fwd_ties, host, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("block", [32, 1])
def test_rotated_quantizer_bit_exact(d, block):
    from bit_causal_flash_amd import flamia as F
    log("case rotated quantizer d=%d block=%d" % (d, block))
    rng = np.random.default_rng(21)
    T, H = 300, 3
    x = rng.standard_normal((T, H, d)).astype(np.float32)
    x[rng.random((T, H, d)) < 0.01] *= 30.0          # outliers
    x[40:50] *= np.float32(1e-3)
    x[60, 1] = 0.0                                    # an all-zero row
    bits = workloads.f32_to_bf16_bits(x)
    cu = np.array([0, 17, 130, 131, 290], np.int32)  # rows 290.. are padding
    mode = (F.FLAMIA_SCALE_PER_TOKEN if block == 1 else F.FLAMIA_SCALE_TOKBLOCK32) | F.FLAMIA_SCALE_ROTATE
    p = F.make_problem(dev(cu), T, H, H, d, 0.0, F.FLAMIA_CAUSAL)
    codes, exps = F.quantize(p, dev(bits.view(np.int16)), H, mode)
    rc, re = oracle.quantize_rotated(bits, cu, block=block)
    assert np.array_equal(host(codes), rc), "codes"
    assert np.array_equal(host(exps), re), "exponents"


CASES = [
    # name, lens, capacity, Hq, Hkv, d
    ("had_gqa_d128", [190, 333, 40], 600, 4, 2, 128),
    ("had_mha_d64", [256, 97, 5], 380, 2, 2, 64),
    # 8 q heads per kv head: the backward splits its longest tickets, and the
    # pair kernel un-rotates dK after adding the halves
    ("had_split_gqa_d128", [700, 300, 520], 1536, 8, 1, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rotated_forward_backward(case):
    import torch
    from bit_causal_flash_amd import flamia as F
    name, lens, cap, Hq, Hkv, d = case
    log("case %s" % name)
    w = workloads.make(name, 7, cap, lens, Hq, Hkv, d)
    flags = F.FLAMIA_CAUSAL | F.FLAMIA_HADAMARD
    p = F.make_problem(dev(w.cu.astype(np.int32)), w.T, Hq, Hkv, d, 0.0, flags)
    x = {n: dev(getattr(w, n).view(np.int16)) for n in ("q", "k", "v", "do")}
    rot = F.FLAMIA_SCALE_TOKBLOCK32 | F.FLAMIA_SCALE_ROTATE
    q = F.quantize(p, x["q"], Hq, rot)
    k = F.quantize(p, x["k"], Hkv, rot)
    v = F.quantize(p, x["v"], Hkv)
    o, lse = F.attn_fwd(p, q, k, v)
    dq, dk, dv, ws = F.attn_bwd(p, q, k, v, o, lse, x["do"].view(torch.bfloat16))
    torch.cuda.synchronize()
    rq = oracle.quantize_rotated(w.q, w.cu)
    rk = oracle.quantize_rotated(w.k, w.cu)
    rv = oracle.quantize(w.v, w.cu)
    for tag, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert np.array_equal(host(got[0]), ref[0]) and np.array_equal(host(got[1]), ref[1]), tag
    s = oracle.default_scale(d) / d
    ops = oracle.Operands.from_codes(rq, rk, rv)
    O, L = oracle.attn_fwd(w.cu, ops, scale=s, mode=oracle.MODE_TILED, kblock=64)
    ties = fwd_ties(w.cu, ops, scale=s)
    Og = host(o).view(np.uint16)
    check_fwd(Og.reshape(-1, d), host(lse).T.ravel(), O.reshape(-1, d), L.T.ravel(),
              ties.transpose(1, 0, 2).reshape(-1, 2), tag=name)
    # both quantized routes approximate the same attention: against the FP64
    # attention of the unquantized bf16 inputs
    exact = oracle.Operands(*(oracle.bf16_to_float(getattr(w, n)) for n in ("q", "k", "v")))
    Oe, _ = oracle.attn_fwd(w.cu, exact, mode=oracle.MODE_REFERENCE)
    plain = oracle.Operands.from_codes(*(oracle.quantize(getattr(w, n), w.cu) for n in ("q", "k", "v")))
    O0, _ = oracle.attn_fwd(w.cu, plain, mode=oracle.MODE_TILED, kblock=64)
    c_rot = metrics_cos(oracle.bf16_to_float(Og).ravel(), Oe.ravel())
    c_plain = metrics_cos(O0.ravel(), Oe.ravel())
    log("%s: cosine against the unquantized attention: rotated %.6f, unrotated %.6f" % (name, c_rot, c_plain))
    assert c_rot > 0.995
    # backward: prep at the same effective scale, bit-exact
    T = w.T
    Lay = F.flamia_attn_bwd_workspace_layout(p)
    wsn = host(ws)
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, Og, rk[1], rv[1], Hkv, scale=s)
    assert np.array_equal(wsn[Lay.do_codes:Lay.do_codes + T * Hq * d].reshape(T, Hq, d), gc)
    assert np.array_equal(wsn[Lay.dq_prescale:Lay.dq_prescale + Hq * T].view(np.int8).reshape(Hq, T)
                          .astype(np.int32), kpre)
    G = oracle.dequantize(gc, ge)
    lse64 = host(lse).astype(np.float64)
    # compared in the rotated frame the oracle computes in: the GPU's dQ and
    # dK are dQ_r H and dK_r H, and H H = d I, so dQ_r = dQ H / d exactly in
    # real arithmetic
    Hm = oracle.hadamard_matrix(d)
    Backward(w.cu, ops, G, D, lse64, kpre=kpre, scale=s).check(
        dict(dQ=host(dq).view(np.uint16), dK=host(dk).view(np.uint16), dV=host(dv).view(np.uint16)),
        name, frame=lambda x: x @ Hm / d)
    n = int(w.cu[-1])
    for t in (dq, dk, dv):
        assert np.all(host(t)[n:] == 0)


def metrics_cos(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))
