"""Causality and determinism of the HIP path (review section 10, "Turn
prefix independence into a tested contract").

Perturbing the inputs of a later document-local 32-token block must leave the
forward outputs (O, LSE) of every query in earlier blocks bit-identical, and,
with FLAMIA_DETERMINISTIC, their dQ too; the default atomic backward is
checked against its own run-to-run spread.  A negative control perturbs a
different document and moves it by a non-multiple of 32 rows."""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import check_grad, log, oracle_operands, run_gpu

pytestmark = pytest.mark.gpu

DET = 1 | 8  # causal | deterministic


def _perturb(x, rows, factor):
    f = workloads.bf16_bits_to_f32(x).copy()
    f[rows] *= np.float32(factor)
    return workloads.f32_to_bf16_bits(f)


def _make(lens, cap, Hq=4, Hkv=2, d=128, seed=5):
    return workloads.make("causal", seed, cap, lens, Hq, Hkv, d)


def test_deterministic_backward_is_bitwise_repeatable():
    w = _make([300, 190], 500)
    a = run_gpu(w, flags=DET)
    b = run_gpu(w, flags=DET)
    for k in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.array_equal(a[k], b[k]), k


def test_deterministic_dq_parity():
    w = _make([257, 64, 130], 460, Hq=4, Hkv=1, d=64)
    g = run_gpu(w, flags=DET)
    q, k, v = oracle_operands(w)
    ops = oracle.Operands.from_codes(q, k, v)
    gc, ge, D, _ = oracle.bwd_prep(w.cu, w.do, g["O"], k[1], v[1], w.Hkv)
    G = oracle.dequantize(gc, ge)
    lse = g["LSE"].astype(np.float64)
    dQ, tq, _, aq = oracle.bwd_dq(w.cu, ops, G, D, lse, want_flags=True)
    # FP32 accumulation: no FP16 accumulation allowance
    check_grad(g["dQ"], dQ, "deterministic dQ", tq, absm=aq)
    assert np.all(g["dQ"][int(w.cu[-1]):] == 0)


@pytest.mark.parametrize("block", [1, 3])
def test_later_block_perturbation_leaves_earlier_queries_bit_identical(block):
    lens, cap = [200, 150], 360
    w0 = _make(lens, cap)
    w1 = _make(lens, cap)
    rows = slice(32 * block, 32 * block + 32)
    for name in ("q", "k", "v", "do"):
        setattr(w1, name, _perturb(getattr(w1, name), rows, 8.0))
    a, b = run_gpu(w0, flags=DET), run_gpu(w1, flags=DET)
    hi = 32 * block
    assert np.array_equal(a["O"][:hi], b["O"][:hi])
    assert np.array_equal(a["LSE"][:, :hi], b["LSE"][:, :hi])
    assert np.array_equal(a["dQ"][:hi], b["dQ"][:hi])
    assert np.array_equal(a["kpre"][:, :hi], b["kpre"][:, :hi])
    # the perturbed block itself did change
    assert not np.array_equal(a["O"][rows], b["O"][rows])
    # the other document is untouched entirely
    for k in ("O", "dQ", "dK", "dV"):
        assert np.array_equal(a[k][200:350], b[k][200:350]), k
    # default (atomic FP16) backward: earlier dQ rows differ from the
    # unperturbed run no more than two unperturbed runs differ from each other
    a1, a2, b1 = run_gpu(w0), run_gpu(w0), run_gpu(w1)
    assert np.array_equal(a1["O"][:hi], b1["O"][:hi])
    fa1 = oracle.bf16_to_float(a1["dQ"][:hi])
    spread = np.abs(fa1 - oracle.bf16_to_float(a2["dQ"][:hi])).max()
    change = np.abs(fa1 - oracle.bf16_to_float(b1["dQ"][:hi])).max()
    ulp = 2.0 ** -7 * np.abs(fa1).max()
    log("atomic dQ: run-to-run spread %.3g, change under the perturbation %.3g" % (spread, change))
    assert change <= max(spread, ulp)


def test_other_document_negative_control():
    # perturb the third document and move it by 5 rows (not a multiple of 32)
    w0 = _make([77, 40, 60], 200)
    w1 = _make([77, 45, 60], 200)
    for name in ("q", "k", "v", "do"):
        setattr(w1, name, _perturb(getattr(w1, name), slice(122, 182), 30.0))
    a, b = run_gpu(w0, flags=DET), run_gpu(w1, flags=DET)
    for k in ("O", "dQ", "dK", "dV"):
        assert np.array_equal(a[k][:77], b[k][:77]), k
    assert np.array_equal(a["LSE"][:, :77], b["LSE"][:, :77])
