"""Pins of the FP16 dQ accumulation model and of the sequence-wide prescale
control (CPU only).

The dQ partials are reduced in FP16 after a power-of-two boost ([R] section
4 "Forward locality and backward locality differ"; [K] section 3.3).  The
method sizes the boost per query row from what the row may see; the
negative control sizes it from sequence-wide maxima, so that a later outlier
moves the FP16 rounding of earlier rows ([K] section 3.3 quotes a change of
up to 5e-4 of the row's largest entry in its Appendix A.4).  Powers of two
commute with FP16 rounding in the normal range, so the leak runs through the
subnormal range: a smaller boost pushes small entries below 2^-14."""
import numpy as np
import pytest

import oracle
import workloads
from tests.oracle_helpers import mirror_pipeline, small_problem


def test_f16_round_matches_numpy_binary16():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(20000) * np.exp2(rng.uniform(-30.0, 17.0, 20000))
    special = [1.0 + 2.0 ** -11,          # tie -> 1.0 (even)
               1.0 + 3 * 2.0 ** -11,      # tie -> 1 + 2^-9 (even)
               2.0 ** -25,                # tie between 0 and the smallest subnormal -> 0
               3 * 2.0 ** -25,            # tie -> 2^-23
               2.0 ** -14 - 2.0 ** -25,   # largest subnormal region tie -> 2^-14
               65504.0, 65519.99, 65520.0, -65520.0, 1e6, 0.0, -0.0]
    x = np.concatenate([x, np.array(special)])
    got = np.array([oracle.f16_round(v) for v in x])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def _with_prescale(w, seq):
    r = mirror_pipeline(w)
    kp = (oracle.bwd_prescale_seq(w.cu, r["ge"], r["k"][1], r["v"][1], w.Hkv, w.d)
          if seq else r["kpre"])
    lse = r["LSE"].astype(np.float64)
    dQ, dq16 = oracle.bwd_dq(w.cu, r["ops"], r["G"], r["D"], lse, causal=w.causal, kpre=kp,
                             dq_tile=128)
    return r, kp, dQ, dq16, _tile_partial_magnitudes(w, r, lse)


def _tile_partial_magnitudes(w, r, lse):
    """Per row: the sum over its 128-key tiles of the largest magnitude of
    the tile's dQ partial (scale sum_j dS^_ij K_j over the tile's keys), from
    the oracle's 32x32 blocks."""
    ops, scale = r["ops"], oracle.default_scale(w.d)
    acc = np.zeros((w.T, w.Hq))
    for h in range(w.Hq):
        g = h * w.Hkv // w.Hq
        for b in range(len(w.cu) - 1):
            s0, s1 = int(w.cu[b]), int(w.cu[b + 1])
            for q0 in range(s0, s1, 32):
                n = min(32, s1 - q0)
                part = np.zeros((32, w.d))
                for k0 in range(s0, min(q0 + 32, s1), 32):
                    kn = min(32, s1 - k0)
                    blk = oracle.bwd_block(w.cu, ops, r["G"], r["D"], lse, h, q0, k0,
                                           causal=w.causal)
                    part += scale * blk["dSq"][:, :kn] @ ops.K[k0:k0 + kn, g]
                    if (k0 - s0) // 32 % 4 == 3 or k0 + 32 >= min(q0 + 32, s1):
                        acc[q0:q0 + n, h] += np.abs(part[:n]).max(axis=1)
                        part[:] = 0.0
    return acc


def _scaled_rows(x, rows, factor):
    f = workloads.bf16_bits_to_f32(x).copy()
    f[rows] *= np.float32(factor)
    return workloads.f32_to_bf16_bits(f)


def test_sequence_prescale_rule():
    w = small_problem(51, [100, 70], 2, 1, 32, capacity=180)
    r = mirror_pipeline(w)
    kc = r["kpre"]
    ks = oracle.bwd_prescale_seq(w.cu, r["ge"], r["k"][1], r["v"][1], w.Hkv, w.d)
    ntok = 170
    # one exponent per head for every row of every document, 0 on padding
    for h in range(2):
        assert np.all(ks[h, :ntok] == ks[h, 0])
    assert np.all(ks[:, ntok:] == 0)
    # maxima over more tokens: never a larger boost than the causal rule
    assert np.all(ks[:, :ntok] <= kc[:, :ntok])
    assert np.any(ks[:, :ntok] < kc[:, :ntok])

    # equality case: when the last block of the only document holds the
    # largest dO, K and V exponents, its rows see every maximum
    w2 = small_problem(52, [96], 1, 1, 32)
    for name in ("do", "k", "v"):
        setattr(w2, name, _scaled_rows(getattr(w2, name), slice(64, 96), 32.0))
    r2 = mirror_pipeline(w2)
    ks2 = oracle.bwd_prescale_seq(w2.cu, r2["ge"], r2["k"][1], r2["v"][1], 1, 32)
    assert np.array_equal(ks2[:, 64:], r2["kpre"][:, 64:])
    assert np.all(ks2[:, :64] < r2["kpre"][:, :64])


def test_fp16_model_within_its_rounding_bound():
    w = small_problem(53, [300, 60], 2, 1, 32)
    r, kp, dQ, dq16, acc = _with_prescale(w, seq=False)
    scale = oracle.default_scale(w.d)
    f = int(np.floor(np.log2(scale)))
    assert np.all(np.isfinite(dq16))
    # every step rounds to FP16 once for the boosted partial and once for the
    # running sum: relative 2^-11 of each, or half a subnormal spacing
    pos = np.concatenate([np.arange(0, 300), np.arange(0, 60)])
    ntiles = pos // 128 + 1
    unit = scale * np.exp2(-(kp.T + f))                    # [T][Hq]: one boosted unit, unscaled back
    bound = 2.0 ** -11 * acc * (1.0 + 1.01 * ntiles[:, None]) + ntiles[:, None] * unit * 2.0 ** -24
    err = np.abs(dq16 - dQ).max(axis=2)
    assert np.all(err <= bound)
    # one 128-key tile: the result is one FP16 rounding of the boosted
    # partial (rows of the 60-token document): an FP16 value within half an
    # FP16 step of it.  (The partials are dyadic, so exact ties are common;
    # unscaling dQ by the softmax scale rounds in FP64, hence the slack.)
    rows = slice(300, 360)
    y = dq16[rows] / scale * np.exp2(kp.T[rows] + f)[:, :, None]
    x = dQ[rows] / scale * np.exp2(kp.T[rows] + f)[:, :, None]
    assert np.allclose(y, y.astype(np.float16).astype(np.float64), rtol=1e-13, atol=0.0)
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    step = np.exp2(np.floor(np.log2(ax)) - 10)
    assert np.all(np.abs(y - x) <= 0.5 * step * (1 + 1e-9) + 1e-13 * np.abs(x))


@pytest.mark.parametrize("seq", [False, True])
def test_suffix_outlier_through_the_prescale(seq):
    """Table-5-style probe on the FP16 model: a V row of the last block of a
    later document is raised by 2^12; earlier rows' exact dQ does not move,
    and neither does their FP16-reduced dQ under the per-row rule.  Under
    the sequence-wide rule it does, by at most about an FP16 rounding of the
    row's largest entry."""
    lens, cap = [130, 90], 220
    w0 = small_problem(54, lens, 2, 1, 32, capacity=cap)
    w1 = small_problem(54, lens, 2, 1, 32, capacity=cap)
    w1.v = _scaled_rows(w1.v, slice(200, 201), 4096.0)
    first = 130 + 64            # the perturbed token's block
    r0, kp0, dQ0, q0, _ = _with_prescale(w0, seq)
    r1, kp1, dQ1, q1, _ = _with_prescale(w1, seq)
    assert np.array_equal(dQ0[:first], dQ1[:first])
    if not seq:
        assert np.array_equal(kp0[:, :first], kp1[:, :first])
        assert np.array_equal(q0[:first], q1[:first])
        return
    assert np.all(kp1[:, :first] < kp0[:, :first])
    rowmax = np.abs(dQ0[:first]).max(axis=2, keepdims=True)
    diff = np.abs(q1[:first] - q0[:first])
    # rows whose gradient is exactly zero (each document's first token) stay zero
    assert np.all(diff[np.broadcast_to(rowmax == 0, diff.shape)] == 0)
    rel = np.where(rowmax > 0, diff / np.where(rowmax > 0, rowmax, 1.0), 0.0).max()
    print("sequence-wide prescale: largest change of earlier dQ rows %.3g of the row maximum" % rel)
    assert rel > 0.0
    assert rel < 4e-3
