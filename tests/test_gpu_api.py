"""The PyTorch operator flamia.attn (an autograd Function over the C ABI) and
the agreement of the deterministic and the atomic dQ paths on the quantized
dS they share."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import Backward, check_fwd, dev, fwd_ties, host, log, oracle_operands, \
    run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "deterministic"])
def test_attn_operator_autograd_ragged_gqa(deterministic):
    """torch.autograd.grad through flamia.attn on a ragged GQA case with a
    1-token document and padding rows: O and the gradients against the
    oracle (from the operator's own saved O and LSE), and, deterministic,
    bit-identical to the same calls made through the C ABI directly."""
    import torch
    from bit_causal_flash_amd import flamia as F
    log("case attn operator, deterministic=%s" % deterministic)
    w = workloads.make("op", 11, 600, [190, 1, 333, 60], 4, 2, 128)
    cu = dev(w.cu.astype(np.int32))
    q, k, v = (dev(getattr(w, n).view(np.int16)).view(torch.bfloat16).requires_grad_()
               for n in ("q", "k", "v"))
    dout = dev(w.do.view(np.int16)).view(torch.bfloat16)
    o, lse = F.attn(q, k, v, cu, causal=True, deterministic=deterministic, return_lse=True)
    loss = (o.float() * dout.float()).sum()
    dq, dk, dv = torch.autograd.grad(loss, (q, k, v))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16 and dq.dtype == torch.bfloat16 and dk.shape == k.shape
    qq, kk, vv = oracle_operands(w)
    ops = oracle.Operands.from_codes(qq, kk, vv)
    O, L = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_TILED, kblock=64)
    og = host(o).view(np.uint16)
    check_fwd(og.reshape(-1, w.d), host(lse).T.ravel(), O.reshape(-1, w.d), L.T.ravel(),
              fwd_ties(w.cu, ops).transpose(1, 0, 2).reshape(-1, 2), tag="operator")
    gc, ge, D, kpre = oracle.bwd_prep(w.cu, w.do, og, kk[1], vv[1], w.Hkv)
    G = oracle.dequantize(gc, ge)
    got = dict(dQ=host(dq).view(np.uint16), dK=host(dk).view(np.uint16), dV=host(dv).view(np.uint16))
    Backward(w.cu, ops, G, D, host(lse), kpre=None if deterministic else kpre).check(got, "operator")
    if deterministic:
        g = run_gpu(w, flags=F.FLAMIA_CAUSAL | F.FLAMIA_DETERMINISTIC)
        assert np.array_equal(og, g["O"])
        for name in ("dQ", "dK", "dV"):
            assert np.array_equal(got[name], g[name]), name


def test_attn_operator_rejects_bad_inputs():
    import torch
    from bit_causal_flash_amd import flamia as F
    x = torch.zeros((64, 2, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 64], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        F.attn(x.float(), x, x, cu)
    with pytest.raises(ValueError):
        F.attn(x, x, x, cu.long())
    # a head dim the kernels do not build: the library's status, raised
    y = torch.zeros((64, 2, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(F.FlamiaError):
        F.attn(y, y, y, cu)


@pytest.mark.parametrize("d", [64, 128])
def test_deterministic_and_atomic_dq_share_ds(d):
    """Documents of at most one 128-key tile: each dQ row is one partial, so
    the atomic path's dQ is the deterministic path's FP32 product after one
    FP16 rounding of the prescaled partial (2^-11 relative), so their bf16
    outputs lie at most one bf16 step apart (2^-7 relative).  They agree that
    closely only if they quantized dS to the same codes and block exponents:
    one E4M3 step of a dS element is 6-12 % of its contribution."""
    from bit_causal_flash_amd import flamia as F
    log("case deterministic vs atomic dQ, d=%d" % d)
    w = workloads.make("onetile", 13, 512, [128, 97, 33, 128, 64, 1, 60], 4, 2, d)
    a = run_gpu(w)
    b = run_gpu(w, flags=F.FLAMIA_CAUSAL | F.FLAMIA_DETERMINISTIC)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["kpre"], b["kpre"])
    ga, gb = oracle.bf16_to_float(a["dQ"]), oracle.bf16_to_float(b["dQ"])
    # each document's first row is 0 in exact arithmetic and FP32 residue
    # here: elements are compared at no less than 2^-12 of the largest one
    scale = np.maximum(np.abs(gb), 2.0 ** -12 * np.abs(gb).max())
    rel = np.abs(ga - gb) / scale
    bad = rel > 2.0 ** -6
    log("largest difference %.3g of the element; elements beyond 2^-6: %d of %d"
        % (rel.max(), int(bad.sum()), bad.size))
    assert not bad.any()
    for name in ("dK", "dV"):
        assert np.array_equal(a[name], b[name]), name
