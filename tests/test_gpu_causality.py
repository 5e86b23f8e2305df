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
from tests.gpu_helpers import Backward, log, oracle_operands, run_gpu

pytestmark = pytest.mark.gpu

DET = 1 | 8  # causal | deterministic
SEQC = 1 | 32  # causal | sequence-wide dQ prescale (negative control)


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


def test_split_backward_is_bitwise_repeatable():
    """Long tickets split in two (8 q heads per kv head): dK and dV are the
    pair kernel's sum of the halves' slots, so they repeat bitwise in both
    modes; with FLAMIA_DETERMINISTIC so does everything else."""
    w = workloads.make("split", 3, 1536, [700, 300, 520], 8, 1, 128)
    a, b = run_gpu(w), run_gpu(w)
    for k in ("O", "LSE", "dK", "dV"):
        assert np.array_equal(a[k], b[k]), k
    a, b = run_gpu(w, flags=DET), run_gpu(w, flags=DET)
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
    # FP32 accumulation in registers: the reference is the FP64 dQ (no FP16
    # accumulation model)
    Backward(w.cu, ops, G, D, lse).check(dict(dQ=g["dQ"]), "deterministic dQ")
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


FLOOR = 0x200  # FLAMIA_SCALE_FLOOR_CONTROL


@pytest.mark.parametrize("per_token", [False, True])
def test_floor_rule_control_codes_bit_exact(per_token):
    """The test-only floor rule (jaehun.me section 2) on the GPU, including
    block maxima that it clips, against the oracle's rule 1."""
    import torch
    from bit_causal_flash_amd import flamia as F
    from tests.gpu_helpers import dev, host
    rng = np.random.default_rng(13)
    T, H, d = 200, 2, 64
    x = rng.standard_normal((T, H, d)).astype(np.float32)
    x[5, 0, 3] = 15.0      # mantissa 1.875: clipped by the floor rule
    x[77, 1, 9] = -30.0
    x[100:104] *= np.float32(1e-30)
    bits = workloads.f32_to_bf16_bits(x)
    cu = np.array([0, 45, 190], np.int32)
    log("case floor rule per_token=%s" % per_token)
    p = F.make_problem(dev(cu), T, H, H, d, 0.0, F.FLAMIA_CAUSAL)
    mode = (F.FLAMIA_SCALE_PER_TOKEN if per_token else 0) | FLOOR
    codes, exps = F.quantize(p, dev(bits.view(np.int16)), H, mode)
    torch.cuda.synchronize()
    rc, re = oracle.quantize(bits, cu, block=1 if per_token else 32, rule=1)
    assert np.array_equal(host(codes), rc) and np.array_equal(host(exps), re)


def _value_leak(rule_mode):
    # one document, d = 64; V of token 3 holds 480 and token 20 of the same
    # block is raised to 900; all other values are integers in [1, 16]
    T, d = 32, 64
    rng = np.random.default_rng(6)
    q = np.zeros((T, 1, d), np.float32)
    k = np.zeros((T, 1, d), np.float32)
    v = rng.integers(1, 17, (T, 1, d)).astype(np.float32)
    v[3, 0, 0] = 480.0
    do = np.ones((T, 1, d), np.float32)
    cu = np.array([0, T], dtype=np.int32)
    v2 = v.copy()
    v2[20, 0, 0] = 900.0
    out = []
    for vv in (v, v2):
        w = workloads.Workload("leak", T, cu, 1, 1, d, workloads.FLAG_CAUSAL,
                               workloads.f32_to_bf16_bits(q), workloads.f32_to_bf16_bits(k),
                               workloads.f32_to_bf16_bits(vv), workloads.f32_to_bf16_bits(do))
        out.append(run_gpu(w, flags=DET, scale_mode=rule_mode))
    return out


def test_floor_rule_positive_control_leaks_and_ceil_rule_does_not():
    """Token 20 of a block moves query 5's output under the floor rule (its
    value 480 is clipped to 448 before and exact after), never under the
    method's conservative rule."""
    a, b = _value_leak(FLOOR)
    assert not np.array_equal(a["O"][5], b["O"][5])
    a, b = _value_leak(0)
    assert np.array_equal(a["O"][:20], b["O"][:20])
    assert np.array_equal(a["LSE"][:, :20], b["LSE"][:, :20])
    assert np.array_equal(a["dQ"][:20], b["dQ"][:20])


def _rel_change(a, b, rows):
    a = oracle.bf16_to_float(a[rows]).reshape(len(range(*rows.indices(a.shape[0]))), -1)
    b = oracle.bf16_to_float(b[rows]).reshape(a.shape)
    den = np.maximum(np.abs(a).max(axis=1), 1e-30)
    return float((np.abs(a - b).max(axis=1) / den).max())


def test_leak_probe_table5():
    """A Table-5-style probe (review section 9, "Separate numerical closeness,
    invariance, and training quality"): a later token of a block is raised so
    that the block's maximum, and with it the scale, changes; report the
    largest relative change of the outputs and dQ rows of every earlier
    query.  The block's earlier maximum (15 = 1.875 * 2^3) is clipped by the
    floor rule at the old scale and exact at the new one.  Method rule: earlier
    blocks bit-identical, earlier rows of the same block unchanged up to the
    subnormal lattice shift; floor rule (control): a visible change; the
    exact option (per-token scales): every earlier row bit-identical."""
    lens, cap = [300, 190], 500
    res = {}
    for tag, mode in (("ceil", 0), ("floor", FLOOR), ("exact", 1)):
        flags = (1 | 2) if tag == "exact" else DET  # the exact option: per-token scales
        runs = []
        for perturb in (False, True):
            w = _make(lens, cap, Hq=2, Hkv=2, d=128)
            for name in ("k", "v"):
                f = workloads.bf16_bits_to_f32(getattr(w, name)).copy()
                f[70, :, 0] = 15.0
                if perturb:
                    f[84, :, 0] = 31.0
                setattr(w, name, workloads.f32_to_bf16_bits(f))
            runs.append(run_gpu(w, flags=flags, scale_mode=mode))
        a, b = runs
        res[tag] = {"O earlier blocks": _rel_change(a["O"], b["O"], slice(0, 64)),
                    "O same block": _rel_change(a["O"], b["O"], slice(70, 84))}
        if tag != "exact":  # its dQ is accumulated by atomics: not run-to-run exact
            res[tag].update({"dQ earlier blocks": _rel_change(a["dQ"], b["dQ"], slice(0, 64)),
                             "dQ same block": _rel_change(a["dQ"], b["dQ"], slice(70, 84))})
        log("leak probe, %s rule: %s" % (tag, res[tag]))
    assert res["ceil"]["O earlier blocks"] == 0.0 and res["ceil"]["dQ earlier blocks"] == 0.0
    assert res["floor"]["O earlier blocks"] == 0.0
    assert res["floor"]["O same block"] > 1e-3
    assert res["ceil"]["O same block"] <= 1e-2 * res["floor"]["O same block"]
    # per-token scales: no earlier output depends on a later token at all
    assert res["exact"]["O earlier blocks"] == 0.0 and res["exact"]["O same block"] == 0.0


def test_sequence_prescale_control():
    """The sequence-wide dQ prescale, a test-only negative control (review
    section 4 "Forward locality and backward locality differ"; jaehun.me
    section 3.3).  Its exponents are bit-exact against the oracle's rule.  A
    V outlier in the last block of a later document lowers them for every
    earlier row, while the method's per-row exponents of those rows stay put.
    dQ under the control keeps parity: only its FP16 rounding moves.  (The
    size of that move is measured on the oracle's FP16 accumulation model:
    on the GPU it is as small as the run-to-run spread of the atomic order.)"""
    lens, cap = [130, 90], 240
    first = 130 + 64  # the perturbed token's block
    runs = {}
    for perturb in (False, True):
        w = _make(lens, cap, Hq=2, Hkv=1, d=64, seed=54)
        if perturb:
            w.v = _perturb(w.v, slice(200, 201), 4096.0)
        q, k, v = oracle_operands(w)
        ctl = run_gpu(w, flags=SEQC)
        met = run_gpu(w, flags=1)
        gc, ge, D, kc = oracle.bwd_prep(w.cu, w.do, ctl["O"], k[1], v[1], w.Hkv)
        ks = oracle.bwd_prescale_seq(w.cu, ge, k[1], v[1], w.Hkv, w.d)
        assert np.array_equal(ctl["kpre"].astype(np.int32), ks)
        assert np.array_equal(met["kpre"].astype(np.int32), kc)
        runs[perturb] = dict(w=w, ctl=ctl, met=met, ops=oracle.Operands.from_codes(q, k, v),
                             G=oracle.dequantize(gc, ge), D=D)
    a, b = runs[False], runs[True]
    assert np.array_equal(a["met"]["kpre"][:, :first], b["met"]["kpre"][:, :first])
    assert np.all(b["ctl"]["kpre"][:, :first] < a["ctl"]["kpre"][:, :first])
    log("sequence-wide prescale: earlier rows' exponent %d -> %d; per-row rule unchanged"
        % (int(a["ctl"]["kpre"][0, 0]), int(b["ctl"]["kpre"][0, 0])))
    w = b["w"]
    Backward(w.cu, b["ops"], b["G"], b["D"], b["ctl"]["LSE"], kpre=b["ctl"]["kpre"]).check(
        dict(dQ=b["ctl"]["dQ"]), "dQ, sequence-wide prescale")
