"""Pins of the oracle's forward against the pages' worked example, brute
force, closed forms and its error bound (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from tests.oracle_helpers import quantized_operands, small_problem


def naive_attention(cu, Q, K, V, scale, causal):
    # textbook full softmax, one row at a time, written independently of the
    # oracle's blockwise recurrence
    T, Hq, d = Q.shape
    Hkv = K.shape[1]
    O = np.zeros_like(Q)
    L = np.full((Hq, T), np.inf)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for h in range(Hq):
            g = h * Hkv // Hq
            for i in range(s0, s1):
                j1 = i + 1 if causal else s1
                s = scale * (K[s0:j1, g] @ Q[i, h])
                m = s.max()
                w = np.exp(s - m)
                O[i, h] = (w / w.sum()) @ V[s0:j1, g]
                L[h, i] = m + math.log(w.sum())
    return O, L


def test_two_block_worked_example(golden):
    g = golden("online_softmax_two_blocks.json")
    scores = [x for blk in g["scores"] for x in blk]
    values = [x for blk in g["values"] for x in blk]
    n = len(scores)
    # one document of n tokens, d = 1, scale 1: query rows all 1, key j holds
    # the score, so the last query sees every score and query 1 only block 1
    Q = np.ones((n, 1, 1))
    K = np.array(scores, dtype=np.float64).reshape(n, 1, 1)
    V = np.array(values, dtype=np.float64).reshape(n, 1, 1)
    cu = np.array([0, n], dtype=np.int32)
    ops = oracle.Operands(Q, K, V)
    O, L, nres = oracle.attn_fwd(cu, ops, scale=1.0, causal=True, mode=oracle.MODE_REFERENCE,
                                 kblock=2, want_rescale=True)
    assert round(O[n - 1, 0, 0], 2) == g["printed"]["result_rounded_2dp"]
    assert max(g["scores"][0]) == g["printed"]["block1_max"]
    # block 2 does not raise the running max: no rescale for the last query
    assert nres[0, n - 1] == 0 and not g["printed"]["block2_needs_rescale"]
    # closed forms of the recurrence's state for this reading
    l1 = math.exp(1 - 3) + 1.0
    assert abs(O[1, 0, 0] - (10 * math.exp(-2) + 20) / l1) < 1e-12
    lf = l1 + math.exp(2 - 3) + math.exp(0 - 3)
    assert abs(L[0, n - 1] - (3 + math.log(lf))) < 1e-12
    # blocks of 2 agree with the single pass (the "blocks of 32 keys agree"
    # statement of the same section, here at block size 2)
    O1, _ = oracle.attn_fwd(cu, ops, scale=1.0, causal=True, mode=oracle.MODE_REFERENCE, kblock=64)
    assert abs(O1[n - 1, 0, 0] - O[n - 1, 0, 0]) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("heads", [(2, 2), (4, 2), (3, 1)])
def test_blockwise_reference_equals_naive(causal, heads):
    Hq, Hkv = heads
    w = small_problem(7, [5, 33, 1, 70], Hq, Hkv, 8, causal=causal, capacity=120)
    q, k, v = quantized_operands(w)
    ops = oracle.Operands.from_codes(q, k, v)
    scale = 0.37
    for kb in (1, 32, 7):
        O, L = oracle.attn_fwd(w.cu, ops, scale=scale, causal=causal, mode=oracle.MODE_REFERENCE,
                               kblock=kb)
        On, Ln = naive_attention(w.cu, ops.Q, ops.K, ops.V, scale, causal)
        assert np.allclose(O, On, rtol=1e-12, atol=1e-12 * np.abs(On).max())
        valid = np.isfinite(Ln)
        assert np.allclose(L[valid], Ln[valid], rtol=1e-12, atol=1e-12)
        assert np.all(np.isinf(L[~valid])) and np.all(O[w.cu[-1]:] == 0)


def test_mirror_equals_reference_when_weights_are_representable():
    # scale ln 2 and integer dot products make every base-2 logit an integer,
    # so every weight 2^(s2 - r) is a power of two in [2^-17, 1] and 256 p,
    # down to 2^-9 (the smallest E4M3 subnormal), is an exact E4M3 value: the
    # microscaled forward must then equal the reference.  Each document's
    # first key has logit 0 and its second -17, so every later row holds
    # both ends: a boost of 128 would round 128 * 2^-17 (a tie) to 0, one of
    # 512 would clip the largest weight to 448 / 512.
    rng = np.random.default_rng(4)
    T, d = 40, 4
    Q = np.zeros((T, 1, d))
    Q[:, 0, 0] = 1.0
    K = np.zeros((T, 1, d))
    K[:, 0, 0] = rng.integers(-17, 1, T)
    cu = np.array([0, 17, 40], dtype=np.int32)
    for s in cu[:-1]:
        K[s, 0, 0], K[s + 1, 0, 0] = 0.0, -17.0
    V = rng.integers(-8, 9, (T, 1, d)).astype(np.float64)
    ops = oracle.Operands(Q, K, V)
    Om, Lm = oracle.attn_fwd(cu, ops, scale=math.log(2), mode=oracle.MODE_ROUNDED)
    Or, Lr = oracle.attn_fwd(cu, ops, scale=math.log(2), mode=oracle.MODE_REFERENCE)
    assert np.allclose(Om, Or, rtol=1e-12, atol=1e-12)
    assert np.allclose(Lm, Lr, rtol=1e-12, atol=1e-12)


def test_first_token_output_is_its_value_exactly():
    # a document's first query sees only its own key: with the rounded
    # normaliser O = P^ V / P^ = V exactly, for any score
    w = small_problem(11, [31, 1, 64, 9], 2, 1, 16, capacity=110, scale_q=3.0)
    q, k, v = quantized_operands(w)
    ops = oracle.Operands.from_codes(q, k, v)
    O, L = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_ROUNDED)
    Ou, _ = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_UNROUNDED)
    firsts = w.cu[:-1]
    differs = 0
    for s in firsts:
        for h in range(2):
            assert np.array_equal(oracle.to_bf16(O[s, h]), oracle.to_bf16(ops.V[s, 0]))
            differs += int(not np.allclose(Ou[s, h], ops.V[s, 0], rtol=1e-9))
    assert differs > 0  # the unrounded normaliser does not have this property


def test_identical_keys_give_the_mean_value():
    rng = np.random.default_rng(8)
    T, d = 50, 8
    Q = rng.standard_normal((T, 2, d))
    K = np.repeat(rng.standard_normal((1, 1, d)), T, axis=0)
    V = rng.standard_normal((T, 1, d))
    cu = np.array([0, 20, 50], dtype=np.int32)
    ops = oracle.Operands(Q, K, V)
    for mode in (oracle.MODE_ROUNDED, oracle.MODE_REFERENCE):
        O, _ = oracle.attn_fwd(cu, ops, mode=mode)
        for b in range(2):
            s0 = cu[b]
            for i in range(s0, cu[b + 1]):
                assert np.allclose(O[i, :], V[s0:i + 1, 0].mean(0), rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    w = small_problem(9, [45, 60], 4, 2, 16, capacity=110)
    q, k, v = quantized_operands(w)
    ops = oracle.Operands.from_codes(q, k, v)
    rep = oracle.Operands(ops.Q, np.repeat(ops.K, 2, axis=1), np.repeat(ops.V, 2, axis=1))
    for mode in (oracle.MODE_ROUNDED, oracle.MODE_REFERENCE):
        O1, L1 = oracle.attn_fwd(w.cu, ops, mode=mode)
        O2, L2 = oracle.attn_fwd(w.cu, rep, mode=mode)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_mirror_within_rounding_bound_of_reference():
    # each probability weight carries at most 2^-4 relative rounding error
    # (normal range) in numerator and normaliser, so per element
    # |O_mirror - O_ref| <= (2^-3 / (1 - 2^-4)) max_j |V_jc| plus a tiny
    # subnormal-weight term
    w = small_problem(12, [100, 57, 200], 2, 2, 32, capacity=360, scale_q=2.0)
    q, k, v = quantized_operands(w)
    ops = oracle.Operands.from_codes(q, k, v)
    Om, _ = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_ROUNDED)
    Or, _ = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_REFERENCE)
    bound = (2.0 ** -3 / (1 - 2.0 ** -4)) * np.abs(ops.V).max() + 1e-3
    assert np.abs(Om - Or).max() <= bound
    # and on typical data it is far inside the bound
    cos = np.dot(Om.ravel(), Or.ravel()) / np.linalg.norm(Om) / np.linalg.norm(Or)
    assert cos > 0.999


def test_tiled_mode_equals_final_reference_on_normal_weights():
    # with every weight exactly representable the tile loop (any tile size)
    # equals the final-reference definition and the FP64 reference
    rng = np.random.default_rng(4)
    T, d = 90, 4
    Q = np.zeros((T, 1, d))
    Q[:, 0, 0] = 1.0
    K = np.zeros((T, 1, d))
    K[:, 0, 0] = rng.integers(-12, 1, T)
    V = rng.integers(-8, 9, (T, 1, d)).astype(np.float64)
    cu = np.array([0, 17, 90], dtype=np.int32)
    ops = oracle.Operands(Q, K, V)
    Or, Lr = oracle.attn_fwd(cu, ops, scale=math.log(2), mode=oracle.MODE_REFERENCE)
    rises = 0
    for kb in (1, 7, 64):
        Ot, Lt, nres = oracle.attn_fwd(cu, ops, scale=math.log(2), mode=oracle.MODE_TILED,
                                       kblock=kb, want_rescale=True)
        assert np.allclose(Ot, Or, rtol=1e-12, atol=1e-12)
        assert np.allclose(Lt, Lr, rtol=1e-12, atol=1e-12)
        rises += int(nres.max())
    assert rises > 0  # the running reference did rise in this data


def test_tiled_mode_differs_only_by_subnormal_weights():
    # per weight the tile loop and the final reference differ by at most half
    # an E4M3 subnormal step (2^-10 of the boosted weight, i.e. 2^-18 of the
    # row reference), so |dl| <= n 2^-18 and |dO| <= n 2^-18 max|V| / l
    w = small_problem(13, [300, 77], 2, 1, 64, capacity=400, scale_q=3.0)
    q, k, v = quantized_operands(w)
    ops = oracle.Operands.from_codes(q, k, v)
    O0, L0 = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_ROUNDED)
    for kb in (64, 128):
        O3, L3 = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_TILED, kblock=kb)
        for b in range(2):
            s, e = int(w.cu[b]), int(w.cu[b + 1])
            n = np.arange(1, e - s + 1)[:, None]
            bound = n * 2.0 ** -18 * np.abs(ops.V).max() * 4
            assert np.all(np.abs(O3[s:e] - O0[s:e]).max(axis=2) <= bound)
        assert np.nanmax(np.abs(L3 - L0)[np.isfinite(L0)]) < 1e-2
    # the first token of each document is still exactly its value row
    O3, _ = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_TILED, kblock=64)
    for s in w.cu[:-1]:
        assert np.array_equal(oracle.to_bf16(O3[s, 0]), oracle.to_bf16(ops.V[s, 0]))
