"""Oracle pins of the Hadamard rotation of the score operands (FLAMIA review
section 3 "Rotation, range, and the alternative" and Algorithm 1 step 02;
jaehun.me section 3.4): the matrix against its textbook construction, the FP32
fast transform against the matrix product, the score identity
(x H)(y H)^T = d x y^T, codes of rotated operands on exactly representable
cases, and the gradient un-rotation against the unrotated reference
backward."""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore")


def _sylvester(d):
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128])
def test_matrix_is_the_sylvester_construction(d):
    H = oracle.hadamard_matrix(d)
    assert np.array_equal(H, _sylvester(d))
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, d * np.eye(d))
    assert np.all(H[0] == 1) and np.all(H[:, 0] == 1)


def _bf16(x):
    return workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("d", [64, 128])
def test_fast_transform_equals_matrix_product_on_exact_inputs(d):
    # small integers: every FP32 partial sum is exact, so the fast transform
    # must equal the FP64 matrix product bit for bit
    rng = np.random.default_rng(0)
    x = rng.integers(-64, 65, size=(7, 3, d)).astype(np.float32)
    got = oracle.hadamard_rotate(_bf16(x))
    ref = x.astype(np.float64) @ oracle.hadamard_matrix(d)
    assert np.array_equal(got.astype(np.float64), ref)
    # a one-hot row rotates into the matching row of H
    e = np.zeros((1, 1, d), dtype=np.float32)
    e[0, 0, 5] = 1.0
    assert np.array_equal(oracle.hadamard_rotate(_bf16(e))[0, 0], oracle.hadamard_matrix(d)[5])


@pytest.mark.parametrize("d", [64, 128])
def test_fast_transform_within_fp32_rounding(d):
    rng = np.random.default_rng(1)
    bits = _bf16(rng.standard_normal((50, 2, d)) * np.exp(rng.standard_normal((50, 2, 1)) * 3))
    x = oracle.bf16_to_float(bits)
    got = oracle.hadamard_rotate(bits).astype(np.float64)
    ref = x @ oracle.hadamard_matrix(d)
    # log2(d) stages, each rounding to FP32 once, on partial sums bounded by sum |x|
    bound = np.log2(d) * 2.0 ** -24 * np.abs(x).sum(axis=-1, keepdims=True)
    assert np.all(np.abs(got - ref) <= bound)


def test_score_identity():
    rng = np.random.default_rng(2)
    for d in (64, 128):
        H = oracle.hadamard_matrix(d)
        x = rng.integers(-9, 10, size=(5, d)).astype(np.float64)
        y = rng.integers(-9, 10, size=(6, d)).astype(np.float64)
        assert np.array_equal((x @ H) @ (y @ H).T, d * (x @ y.T))


@pytest.mark.parametrize("d", [64, 128])
def test_codes_of_rotated_hadamard_rows(d):
    # rows 2^k H[i] rotate into d 2^k e_i: one nonzero value per row, which the
    # conservative exponent then represents exactly
    H = oracle.hadamard_matrix(d).astype(np.float32)
    T = 32
    x = np.stack([H[(3 * t) % d] * np.float32(2.0 ** (t % 5 - 2)) for t in range(T)])[:, None, :]
    cu = np.array([0, T], np.int32)
    codes, exps = oracle.quantize_rotated(_bf16(x), cu, block=1)
    deq = oracle.dequantize(codes, exps)
    for t in range(T):
        want = np.zeros(d)
        want[(3 * t) % d] = d * 2.0 ** (t % 5 - 2)
        assert np.array_equal(deq[t, 0], want)
    # block mode: one exponent for the 32 rows, values still exact (powers of two)
    codes, exps = oracle.quantize_rotated(_bf16(x), cu, block=32)
    deq = oracle.dequantize(codes, exps)
    for t in range(T):
        assert deq[t, 0, (3 * t) % d] == d * 2.0 ** (t % 5 - 2)
        assert np.count_nonzero(deq[t, 0]) == 1


def test_gradient_unrotation_against_unrotated_reference():
    """With exact rotated operands (x H, FP64), the reference backward at
    softmax scale / d gives the gradients dQ_r, dK_r with respect to the
    rotated operands, and unrotate(dQ_r) = dQ_r H = dQ, unrotate(dK_r) = dK of
    the unrotated problem, and the same O, LSE and dV
    (no rounding anywhere: oracle reference modes)."""
    rng = np.random.default_rng(3)
    d, Hq, Hkv = 64, 4, 2
    cu = np.array([0, 40, 97, 130], np.int32)
    T = int(cu[-1])
    Q, K, V = (rng.standard_normal((T, h, d)) for h in (Hq, Hkv, Hkv))
    G = rng.standard_normal((T, Hq, d)) * 0.1
    H = oracle.hadamard_matrix(d)
    s = oracle.default_scale(d)
    plain = oracle.Operands(Q, K, V)
    rot = oracle.Operands(Q @ H, K @ H, V)
    O, L = oracle.attn_fwd(cu, plain, scale=s, mode=oracle.MODE_REFERENCE)
    Or, Lr = oracle.attn_fwd(cu, rot, scale=s / d, mode=oracle.MODE_REFERENCE)
    assert np.allclose(Or, O, rtol=1e-10, atol=1e-12) and np.allclose(Lr, L, rtol=1e-12, atol=1e-12)
    D = np.einsum("thc,thc->ht", G, O)
    dQ = oracle.bwd_dq(cu, plain, G, D, L, scale=s, mode=1)
    dK, dV = oracle.bwd_dkdv(cu, plain, G, D, L, scale=s, mode=1)
    dQr = oracle.bwd_dq(cu, rot, G, D, L, scale=s / d, mode=1)
    dKr, dVr = oracle.bwd_dkdv(cu, rot, G, D, L, scale=s / d, mode=1)
    tol = dict(rtol=1e-9, atol=1e-12)
    assert np.allclose(oracle.unrotate(dQr), dQ, **tol)
    assert np.allclose(oracle.unrotate(dKr), dK, **tol)
    assert np.allclose(dVr, dV, **tol)
    # plausible mistakes (a stray 1 / d, or no un-rotation at all) are caught
    assert not np.allclose(oracle.unrotate(dQr) / d, dQ, **tol)
    assert not np.allclose(dQr, dQ, **tol)
