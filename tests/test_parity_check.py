"""The gradient acceptance of the GPU tests, exercised on the CPU with the
oracle standing in for the GPU: its own result passes, a planted error
fails, and a result that took another valid rounding of a near-midpoint dS
element passes only through the re-check against that alternative."""
import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_helpers
from tests.gpu_helpers import Backward
from tests.oracle_helpers import mirror_pipeline, small_problem


@pytest.fixture()
def problem():
    # K outliers (x20 on 2 % of the entries) give this small case
    # near-midpoint dS elements whose other rounding moves a row by more than
    # 5e-2 at the GPU's evaluation error
    w = small_problem(63, [150, 90], 2, 1, 32, capacity=250, do_std=0.5)
    k = workloads.bf16_bits_to_f32(w.k).copy()
    k[np.random.default_rng(63).random(k.shape) < 0.02] *= np.float32(20.0)
    w.k = workloads.f32_to_bf16_bits(k)
    r = mirror_pipeline(w)
    bw = Backward(w.cu, r["ops"], r["G"], r["D"], r["LSE"])
    return w, r, bw


def _bits(x):
    return oracle.to_bf16(x)


def test_the_oracles_own_result_passes(problem):
    w, r, bw = problem
    out = bw.check(dict(dQ=_bits(r["dQ"]), dK=_bits(r["dK"]), dV=_bits(r["dV"])), "self")
    for k in ("dQ", "dK", "dV"):
        assert out[k]["beyond"] == 0


def test_a_planted_error_fails(problem):
    w, r, bw = problem
    dQ = r["dQ"].copy()
    t = 100
    dQ[t, 1] *= 1.1
    with pytest.raises(AssertionError):
        bw.check(dict(dQ=_bits(dQ)), "planted")


def test_another_valid_rounding_passes_through_the_recheck(problem):
    w, r, bw = problem
    ops, scale = r["ops"], oracle.default_scale(w.d)
    # the near-midpoint element whose other rounding moves its row the most
    best = None
    for h in range(w.Hq):
        for q0 in oracle.doc_blocks(w.cu):
            i, j, lo, hi = oracle.dq_ranges(w.cu, ops, r["G"], r["D"], r["LSE"], h, int(q0),
                                            gpu_helpers.NOISE)
            for n in range(i.size):
                x = hi[n] if abs(hi[n]) >= abs(lo[n]) else lo[n]
                delta = x * scale * ops.K[j[n], h * w.Hkv // w.Hq]
                den = max(np.abs(r["dQ"][i[n], h]).max(), 1e-3 * np.abs(r["dQ"]).max())
                rel = np.abs(delta).max() / den
                if best is None or rel > best[0]:
                    best = (rel, i[n], h, delta)
    rel, t, h, delta = best
    assert rel > 0.1  # the case moves its row beyond the 5e-2 tolerance
    dQ = r["dQ"].copy()
    dQ[t, h] += delta
    out = bw.check(dict(dQ=_bits(dQ)), "alternative")
    assert out["dQ"]["beyond"] >= 1
    assert out["dQ"]["resolved_by_alternative"] == out["dQ"]["beyond"]
    # the same move with the re-check switched off fails
    with pytest.raises(AssertionError):
        gpu_helpers.check_grad(_bits(dQ), r["dQ"], "no alternatives")
