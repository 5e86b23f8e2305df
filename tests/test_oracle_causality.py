"""The suffix-perturbation contract on the oracle itself (CPU only).

Protocol (review section 10, "Turn prefix independence into a tested
contract"): perturb the inputs of a later document-local 32-token block and
require the outputs of every query in earlier blocks to stay bit-identical; a
positive control crosses a scale-exponent threshold under the floor rule, and
a negative control perturbs another document while moving its physical
offset by a non-multiple of 32."""
import numpy as np

import oracle
import workloads
from tests.oracle_helpers import mirror_pipeline, small_problem


def _perturb_block(x, rows, factor=8.0, rng=None):
    f = workloads.bf16_bits_to_f32(x).copy()
    if rng is None:
        f[rows] *= np.float32(factor)
    else:
        f[rows] = rng.standard_normal(f[rows].shape).astype(np.float32) * np.float32(factor)
    return workloads.f32_to_bf16_bits(f)


def _check_prefix(r0, r1, hi, per_token=False):
    assert np.array_equal(r0["O"][:hi], r1["O"][:hi])
    assert np.array_equal(r0["LSE"][:, :hi], r1["LSE"][:, :hi])
    assert np.array_equal(r0["dQ"][:hi], r1["dQ"][:hi])
    assert np.array_equal(r0["kpre"][:, :hi], r1["kpre"][:, :hi])
    assert np.array_equal(r0["D"][:, :hi], r1["D"][:, :hi])


def test_later_block_perturbation_leaves_earlier_queries_bit_identical():
    rng = np.random.default_rng(5)
    w0 = small_problem(41, [130, 45], 2, 1, 32, capacity=180)
    r0 = mirror_pipeline(w0)
    for blk, redraw in ((2, False), (1, True), (3, False)):
        w1 = small_problem(41, [130, 45], 2, 1, 32, capacity=180)
        rows = slice(32 * blk, 32 * blk + 32)
        for name in ("q", "k", "v", "do"):
            setattr(w1, name, _perturb_block(getattr(w1, name), rows,
                                             rng=rng if redraw else None))
        r1 = mirror_pipeline(w1)
        _check_prefix(r0, r1, 32 * blk)
        # the perturbation did change the perturbed block's own outputs
        assert not np.array_equal(r0["O"][rows], r1["O"][rows])


def test_per_token_option_is_exact_inside_a_block():
    # with per-token operand scales and per-row dS exponents, a perturbation
    # of later tokens inside the same block leaves earlier rows bit-identical
    w0 = small_problem(42, [64], 1, 1, 16, capacity=64)
    r0 = mirror_pipeline(w0, block=1, per_row_ds=True)
    w1 = small_problem(42, [64], 1, 1, 16, capacity=64)
    for name in ("q", "k", "v", "do"):
        setattr(w1, name, _perturb_block(getattr(w1, name), slice(45, 64), factor=50.0))
    r1 = mirror_pipeline(w1, block=1, per_row_ds=True)
    _check_prefix(r0, r1, 45)


def _value_leak_case(rule):
    # one document, d = 4; V of token 3 holds 480 and a later token of the same
    # block is raised to 900; all other values are integers in [1, 16], so no
    # value sits near the subnormal boundary at either scale
    T, d = 32, 4
    rng = np.random.default_rng(6)
    q = np.zeros((T, 1, d), np.float32)
    k = np.zeros((T, 1, d), np.float32)
    v = rng.integers(1, 17, (T, 1, d)).astype(np.float32)
    v[3, 0, 0] = 480.0
    do = np.ones((T, 1, d), np.float32)
    cu = np.array([0, T], dtype=np.int32)

    def run(vv):
        w = workloads.Workload("leak", T, cu, 1, 1, d, workloads.FLAG_CAUSAL,
                               workloads.f32_to_bf16_bits(q), workloads.f32_to_bf16_bits(k),
                               workloads.f32_to_bf16_bits(vv), workloads.f32_to_bf16_bits(do))
        return mirror_pipeline(w, rule=rule)

    v2 = v.copy()
    v2[20, 0, 0] = 900.0
    return run(v), run(v2)


def test_floor_rule_positive_control_leaks_and_ceil_rule_does_not():
    a, b = _value_leak_case(rule=1)
    # query 5 sees token 3 but not token 20; under the floor rule its output moves
    assert not np.array_equal(a["O"][5], b["O"][5])
    a, b = _value_leak_case(rule=0)
    assert np.array_equal(a["O"][:20], b["O"][:20])


def test_other_document_negative_control():
    # perturb the third document and move it by 5 rows (not a multiple of 32)
    # by lengthening the second: the first document's results are unchanged
    lens0, lens1 = [77, 40, 60], [77, 45, 60]
    w0 = small_problem(43, lens0, 2, 2, 16, capacity=190)
    w1 = small_problem(43, lens1, 2, 2, 16, capacity=190)
    for name in ("q", "k", "v", "do"):
        setattr(w1, name, _perturb_block(getattr(w1, name), slice(122, 182), factor=30.0))
    r0, r1 = mirror_pipeline(w0), mirror_pipeline(w1)
    for key in ("O", "dQ", "dK", "dV"):
        assert np.array_equal(r0[key][:77], r1[key][:77]), key
    assert np.array_equal(r0["LSE"][:, :77], r1["LSE"][:, :77])
