"""Pins of the oracle's backward: finite differences, the centred-gradient
identities, closed-form special cases and the dQ prescale bound (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests.oracle_helpers import mirror_pipeline, small_problem


def _ref_forward(cu, Q, K, V, scale, causal):
    ops = oracle.Operands(Q, K, V)
    return oracle.attn_fwd(cu, ops, scale=scale, causal=causal, mode=oracle.MODE_REFERENCE)


@pytest.mark.parametrize("causal", [True, False])
def test_reference_backward_matches_finite_differences(causal):
    rng = np.random.default_rng(21)
    cu = np.array([0, 5, 12], dtype=np.int32)
    T, Hq, Hkv, d, scale = 14, 2, 1, 4, 0.6
    Q = rng.standard_normal((T, Hq, d))
    K = rng.standard_normal((T, Hkv, d))
    V = rng.standard_normal((T, Hkv, d))
    G = rng.standard_normal((T, Hq, d))
    O, L = _ref_forward(cu, Q, K, V, scale, causal)
    D = np.einsum("thc,thc->ht", G, O)
    ops = oracle.Operands(Q, K, V)
    dQ = oracle.bwd_dq(cu, ops, G, D, L, scale=scale, causal=causal, mode=oracle.MODE_REFERENCE)
    dK, dV = oracle.bwd_dkdv(cu, ops, G, D, L, scale=scale, causal=causal,
                             mode=oracle.MODE_REFERENCE)

    def loss(Qx, Kx, Vx):
        Ox, _ = _ref_forward(cu, Qx, Kx, Vx, scale, causal)
        return float(np.sum(G * Ox))

    h = 1e-6
    for name, X, grad in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            pos = "QKV".index(name)
            args_p[pos], args_m[pos] = Xp, Xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7 * np.abs(num).max()), name
    assert np.all(dQ[12:] == 0) and np.all(dK[12:] == 0) and np.all(dV[12:] == 0)


def test_centred_row_sums_and_D_identity():
    # sum_j dS_ij = 0 and D_i = sum_j P_ij dP_ij when P, dP and D come from the
    # same reconstruction (the review's centred softmax gradient)
    w = small_problem(22, [70, 41], 2, 1, 16, capacity=111)
    q, k, v = (oracle.quantize(x, w.cu) for x in (w.q, w.k, w.v))
    ops = oracle.Operands.from_codes(q, k, v)
    O, L = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_REFERENCE)
    gc, ge, _, _ = oracle.bwd_prep(w.cu, w.do, oracle.to_bf16(O), k[1], v[1], w.Hkv)
    G = oracle.dequantize(gc, ge)
    D = np.einsum("thc,thc->ht", G, O)
    for h in range(2):
        for b in range(2):
            s0, s1 = int(w.cu[b]), int(w.cu[b + 1])
            for q0 in range(s0, s1, 32):
                row_sum = np.zeros(32)
                row_abs = np.zeros(32)
                pdp = np.zeros(32)
                for k0 in range(s0, min(q0 + 32, s1), 32):
                    blk = oracle.bwd_block(w.cu, ops, G, D, L, h, q0, k0,
                                           mode=oracle.MODE_REFERENCE)
                    row_sum += blk["dS"].sum(1)
                    row_abs += np.abs(blk["dS"]).sum(1)
                    pdp += (blk["P"] * blk["dP"]).sum(1)
                n = min(32, s1 - q0)
                assert np.all(np.abs(row_sum[:n]) <= 1e-12 * np.maximum(row_abs[:n], 1e-300))
                assert np.allclose(pdp[:n], D[h, q0:q0 + n], rtol=1e-12, atol=1e-15)


def test_first_tokens_get_zero_dq_and_single_token_documents():
    w = small_problem(23, [33, 1, 60, 1, 17], 3, 1, 16, capacity=120)
    r = mirror_pipeline(w)
    for s in w.cu[:-1]:
        # O_s is exactly V_s, so D_s equals dP_ss and dS_ss = 0 exactly
        assert np.all(r["dQ"][s] == 0.0)
    for b in np.nonzero(np.diff(w.cu) == 1)[0]:
        s = int(w.cu[b])
        assert np.all(r["dK"][s] == 0.0)
    # reference math: a single-token document has P = 1, so dV = dO^ summed
    # over the group's heads and dK = 0
    ops = r["ops"]
    O, L = oracle.attn_fwd(w.cu, ops, mode=oracle.MODE_REFERENCE)
    D = np.einsum("thc,thc->ht", r["G"], O)
    dK, dV = oracle.bwd_dkdv(w.cu, ops, r["G"], D, L, mode=oracle.MODE_REFERENCE)
    for b in np.nonzero(np.diff(w.cu) == 1)[0]:
        s = int(w.cu[b])
        assert np.allclose(dV[s, 0], r["G"][s].sum(0), rtol=1e-14, atol=0)
        assert np.all(np.abs(dK[s]) <= 1e-14 * np.abs(ops.Q[s]).max())


def test_ds_blocks_use_one_conservative_exponent():
    w = small_problem(24, [80], 1, 1, 16, capacity=80)
    r = mirror_pipeline(w)
    ops, G, D = r["ops"], r["G"], r["D"]
    L = r["LSE"].astype(np.float64)
    for q0, k0 in ((32, 0), (64, 32), (64, 64)):
        blk = oracle.bwd_block(w.cu, ops, G, D, L, 0, q0, k0)
        amax = np.abs(blk["dS"]).max()
        e = oracle.ceil_exponent(amax)
        assert np.abs(blk["dSk"]).max() <= 448 * 2.0 ** e
        nz = blk["dSk"] != 0
        # every quantized entry is an E4M3 value times 2^e
        for val in blk["dSk"][nz]:
            c = oracle.e4m3_encode(val * 2.0 ** -e)
            assert oracle.e4m3_decode(c) * 2.0 ** e == val


def test_dq_prescale_keeps_partials_in_fp16_range():
    # kpre_i is chosen so that every partial sum of dQ_i, boosted by 2^kpre_i,
    # stays at or below 2^14; check it on outlier-heavy data over every
    # 32-key partial and every running prefix of partials
    for seed, (lens, Hq, Hkv, d) in enumerate([([150, 90], 2, 1, 64), ([200], 2, 2, 128)]):
        w = small_problem(30 + seed, lens, Hq, Hkv, d, capacity=sum(lens), do_std=30.0)
        kv = np.asarray(workloads_scale(w.k, 20.0))
        w.k = kv
        r = mirror_pipeline(w)
        ops, G, D = r["ops"], r["G"], r["D"]
        L = r["LSE"].astype(np.float64)
        scale = 1.0 / np.sqrt(d)
        for h in range(Hq):
            g = h * Hkv // Hq
            for b in range(len(lens)):
                s0, s1 = int(w.cu[b]), int(w.cu[b + 1])
                for q0 in range(s0, s1, 32):
                    run = np.zeros((32, d))
                    for k0 in range(s0, min(q0 + 32, s1), 32):
                        blk = oracle.bwd_block(w.cu, ops, G, D, L, h, q0, k0)
                        kn = min(32, s1 - k0)
                        part = scale * blk["dSq"][:, :kn] @ ops.K[k0:k0 + kn, g]
                        run += part
                        n = min(32, s1 - q0)
                        boost = 2.0 ** r["kpre"][h, q0:q0 + n][:, None]
                        assert np.all(np.abs(part[:n]) * boost <= 2.0 ** 14)
                        assert np.all(np.abs(run[:n]) * boost <= 2.0 ** 14)
        assert r["kpre"].min() >= -60 and r["kpre"].max() <= 60


def workloads_scale(x, factor):
    import workloads
    return workloads.f32_to_bf16_bits(workloads.bf16_bits_to_f32(x) * np.float32(factor))


def test_prep_outputs():
    w = small_problem(25, [40, 70], 4, 2, 16, capacity=120)
    r = mirror_pipeline(w)
    # D_i = dO^_i . O_i with the saved bf16 O
    Of = oracle.bf16_to_float(r["O"])
    assert np.allclose(r["D"], np.einsum("thc,thc->ht", r["G"], Of), rtol=1e-13, atol=1e-300)
    # dO codes follow the operand quantizer
    gc, ge = oracle.quantize(w.do, w.cu)
    assert np.array_equal(gc, r["gc"]) and np.array_equal(ge, r["ge"])
    # padding rows
    assert np.all(r["D"][:, 110:] == 0) and np.all(r["kpre"][:, 110:] == 0)


def _representable_problem(T, d, n_lo, seed):
    """One document, one head: Q = e_0 and K_j0 = n_j (an integer in
    [n_lo, 0], K of the document's first key 0 and of its second n_lo), so
    at scale ln 2 every base-2 logit is an integer and, with LSE_i set to
    ln 2 times the row's largest visible logit, P_ij = 2^(n_j - max) is a
    power of two (up to the FP64 rounding of exp) no smaller than 2^n_lo."""
    rng = np.random.default_rng(seed)
    Q = np.zeros((T, 1, d))
    Q[:, 0, 0] = 1.0
    K = np.zeros((T, 1, d))
    K[:, 0, 0] = rng.integers(n_lo, 1, T)
    K[0, 0, 0], K[1, 0, 0] = 0.0, float(n_lo)
    lse = np.zeros((1, T))
    for i in range(T):
        lse[0, i] = math.log(2.0) * K[: i + 1, 0, 0].max()
    return Q, K, lse


def test_probability_operand_boost_is_256_on_powers_of_two():
    # P in {2^0 .. 2^-17}: 256 P runs from 256 down to 2^-9, the smallest E4M3
    # subnormal, so E4M3(256 P) / 256 == P exactly, and the microscaled dV
    # equals the reference one.  A boost of 128 would round 128 * 2^-17 (a
    # tie) to 0; one of 512 would clip P = 1 to 448 / 512.  With every V row
    # equal, dP_ij = D_i for every key, so dS = 0 and dK = dQ = 0 in both modes.
    T, d = 64, 4
    Q, K, lse = _representable_problem(T, d, -17, 31)
    rng = np.random.default_rng(32)
    V = np.repeat(rng.integers(-4, 5, (1, 1, d)).astype(np.float64), T, axis=0)
    G = rng.integers(-3, 4, (T, 1, d)).astype(np.float64)
    D = np.einsum("thc,thc->ht", G, V)
    cu = np.array([0, T], np.int32)
    ops = oracle.Operands(Q, K, V)
    kw = dict(scale=math.log(2.0))
    seen = set()
    for q0 in (0, 32):
        for k0 in range(0, q0 + 1, 32):
            blk = oracle.bwd_block(cu, ops, G, D, lse, 0, q0, k0, **kw)
            vis = blk["P"] > 0
            assert np.allclose(blk["Pq"][vis], blk["P"][vis], rtol=1e-14, atol=0)
            seen |= set(np.round(np.log2(blk["P"][vis])).astype(int).tolist())
            assert np.all(blk["dS"] == 0)
    assert min(seen) == -17 and max(seen) == 0
    dKm, dVm = oracle.bwd_dkdv(cu, ops, G, D, lse, **kw)
    dKr, dVr = oracle.bwd_dkdv(cu, ops, G, D, lse, mode=oracle.MODE_REFERENCE, **kw)
    assert np.allclose(dVm, dVr, rtol=1e-13, atol=1e-13 * np.abs(dVr).max())
    assert np.all(dKm == 0) and np.all(dKr == 0)


def test_microscaled_backward_equals_reference_when_ds_is_representable():
    # P = 2^n, n in [-4, 0], and dP - D a small integer m (|m| <= 15, integer
    # dO and V, D chosen integer): every dS = m 2^n has at most four
    # significant bits, so under the block's conservative exponent (whose
    # maximum is >= 224 after scaling, keeping every entry in E4M3's normal
    # range) each dS is exactly an E4M3 value and the microscaled dK, dQ
    # (and dV) equal the reference ones.  The first document holds a block
    # whose largest |dS| is 15: a floor exponent would scale it to 480 and
    # clip it to 448.
    T, d = 96, 4
    Q, K, lse = _representable_problem(T, d, -4, 33)
    rng = np.random.default_rng(34)
    V = rng.integers(-2, 3, (T, 1, d)).astype(np.float64)
    G = np.zeros((T, 1, d))
    G[:, 0, 0] = 1.0
    # dP_ij = V_j0; D_i an integer so dP - D in [-15, 15]
    D = rng.integers(-2, 3, (1, T)).astype(np.float64)
    V[:, 0, 0] = rng.integers(-13, 14, T)
    V[0, 0, 0], D[0, 0] = 13.0, -2.0                     # dS_00 = P_00 * 15 = 15
    cu = np.array([0, 50, T], np.int32)
    lse[0, 50:] = [math.log(2.0) * K[50: i + 1, 0, 0].max() for i in range(50, T)]
    ops = oracle.Operands(Q, K, V)
    kw = dict(scale=math.log(2.0))
    blk = oracle.bwd_block(cu, ops, G, D, lse, 0, 0, 0, **kw)
    assert np.abs(blk["dS"]).max() == pytest.approx(15.0, rel=1e-14)
    for per_row in (False, True):
        dQm = oracle.bwd_dq(cu, ops, G, D, lse, per_row_ds=per_row, **kw)
        dQr = oracle.bwd_dq(cu, ops, G, D, lse, mode=oracle.MODE_REFERENCE, **kw)
        dKm, dVm = oracle.bwd_dkdv(cu, ops, G, D, lse, per_row_ds=per_row, **kw)
        dKr, dVr = oracle.bwd_dkdv(cu, ops, G, D, lse, mode=oracle.MODE_REFERENCE, **kw)
        for m, r in ((dQm, dQr), (dKm, dKr), (dVm, dVr)):
            assert np.allclose(m, r, rtol=1e-13, atol=1e-13 * np.abs(r).max())
        assert np.abs(dKr).max() > 0 and np.abs(dQr).max() > 0


def _brute_e4m3(y):
    """Nearest E4M3FN value to y by exhaustive search over the 253 finite
    values, ties to the even code (written here independently of the
    oracle's encoder)."""
    vals = []
    for c in range(0x7F):
        E, M = c >> 3, c & 7
        v = (M / 8.0) * 2.0 ** -6 if E == 0 else (1 + M / 8.0) * 2.0 ** (E - 7)
        vals.append((v, c))
    a = min(abs(y), 448.0)
    best = min(vals, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return math.copysign(best[0], y)


def test_microscaled_backward_rounds_p_and_ds_and_stays_within_the_bound():
    # on generic data: P^ is 256 P rounded to the E4M3 lattice over 256, and
    # dS^ is dS over its 32x32 block's conservative exponent rounded to the
    # lattice (both against an exhaustive nearest search); the microscaled
    # dV then differs from the reference dV, by no more than the rounding
    # bound sum_i |P^ - P| |dO_i| <= sum_i (2^-4 P_ij + 2^-18) |dO_i|
    w = small_problem(35, [70, 45], 2, 1, 16, capacity=120)
    r = mirror_pipeline(w)
    ops, G, D = r["ops"], r["G"], r["D"]
    lse = r["LSE"].astype(np.float64)
    blk = oracle.bwd_block(w.cu, ops, G, D, lse, 1, 32, 0)
    vis = blk["P"] > 0
    for p, pq in zip(blk["P"][vis], blk["Pq"][vis]):
        assert pq == _brute_e4m3(256.0 * p) / 256.0
    e = oracle.ceil_exponent(np.abs(blk["dS"]).max())
    assert np.abs(blk["dS"]).max() <= 448 * 2.0 ** e < 2 * np.abs(blk["dS"]).max()
    for s, sq in zip(blk["dS"][vis], blk["dSk"][vis]):
        assert sq == _brute_e4m3(s * 2.0 ** -e) * 2.0 ** e
    dKm, dVm = oracle.bwd_dkdv(w.cu, ops, G, D, lse)
    dKr, dVr = oracle.bwd_dkdv(w.cu, ops, G, D, lse, mode=oracle.MODE_REFERENCE)
    assert np.abs(dVm - dVr).max() > 1e-6 * np.abs(dVr).max()
    # the bound over the keys of the first document (both q heads share the
    # kv head, so dV sums over them)
    bound = np.zeros((70, 16))
    for h in range(2):
        P_all = np.zeros((70, 70))
        for q0 in range(0, 70, 32):
            for k0 in range(0, q0 + 1, 32):
                b = oracle.bwd_block(w.cu, ops, G, D, lse, h, q0, k0)
                nq, nk = min(32, 70 - q0), min(32, 70 - k0)
                P_all[q0:q0 + nq, k0:k0 + nk] = b["P"][:nq, :nk]
        bound += (2.0 ** -4 * P_all + 2.0 ** -18 * (P_all > 0)).T @ np.abs(G[:70, h])
    assert np.all(np.abs(dVm[:70, 0] - dVr[:70, 0]) <= bound * (1 + 1e-12))


@pytest.mark.parametrize("d", [64, 128])
def test_dq_prescale_exponent_is_tight_on_a_worst_case_input(d):
    # The largest dQ a row can reach for given dO, V and K exponents: query 1
    # of a document sees keys 0 and 1 with equal scores (Q_1 alternates
    # +1, -1; K_0 = +448 2^eK, K_1 = -448 2^eK in every feature), so P = 1/2
    # each; V_0 = +448 2^eV, V_1 = -448 2^eV, dO_1 = 448 2^eG in every
    # feature, so O_1 = 0, D_1 = 0, dS = +-P (d 448^2 2^(eG + eV)) and
    # dQ_1 = scale d 448^3 2^(eG + eV + eK) in every feature (the covariance
    # of dP and K under P at its largest), up to the E4M3 rounding of dS.
    # The rule keeps the boosted dQ within (2^11, 2^12] here: one more
    # (or one less) in k_1 would leave that window.  A later block of the
    # same document holds larger K and V exponents, which row 1 may not see:
    # with them k_1 would be 6 smaller.
    T, eG, eV, eK = 64, -3, 2, -1
    f = lambda x: workloads.f32_to_bf16_bits(np.asarray(x, np.float32))
    q = np.zeros((T, 1, d), np.float32)
    q[1, 0, :] = np.where(np.arange(d) % 2 == 0, 1.0, -1.0)
    k = np.zeros((T, 1, d), np.float32)
    v = np.zeros((T, 1, d), np.float32)
    do = np.zeros((T, 1, d), np.float32)
    k[0], k[1] = 448.0 * 2.0 ** eK, -448.0 * 2.0 ** eK
    v[0], v[1] = 448.0 * 2.0 ** eV, -448.0 * 2.0 ** eV
    do[1] = 448.0 * 2.0 ** eG
    k[40], v[40] = 448.0 * 2.0 ** (eK + 3), 448.0 * 2.0 ** (eV + 3)
    w = workloads.make("worst", 0, T, [T], 1, 1, d)
    w.q, w.k, w.v, w.do = f(q), f(k), f(v), f(do)
    r = mirror_pipeline(w)
    assert int(r["ge"][0, 1]) - 127 == eG
    assert int(r["k"][1][0, 1]) - 127 == eK and int(r["v"][1][0, 1]) - 127 == eV
    scale = 1.0 / math.sqrt(d)
    assert np.allclose(r["dQ"][1, 0], r["dQ"][1, 0, 0])           # every feature alike
    exact = scale * d * 448.0 ** 3 * 2.0 ** (eG + eV + eK)
    assert abs(r["dQ"][1, 0, 0]) == pytest.approx(exact * 1.5 / 1.53125, rel=1e-12)
    x = 2.0 ** int(r["kpre"][0, 1]) * np.abs(r["dQ"][1, 0]).max()
    assert 2.0 ** 11 < x <= 2.0 ** 12
