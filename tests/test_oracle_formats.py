"""Pins of the oracle's number formats and token-block quantizer against what
the pages print and what the formats' definitions fix (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def all_finite_bf16():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(h)
    return h[np.isfinite(f)], f[np.isfinite(f)]


def test_e4m3_matches_torch_on_every_bf16_within_range():
    # Exhaustive: every finite bf16 value y with |y| <= 448 encodes exactly as
    # torch's OCP float8_e4m3fn conversion (nearest, ties to even).
    h, f = all_finite_bf16()
    keep = np.abs(f) <= 448.0
    f = f[keep]
    ref = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(y)) for y in f], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(f[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_ties_and_signs(golden):
    fmt = golden("quantizer_examples.json")["format"]
    assert oracle.e4m3_encode(1.0625) == 0x38  # tie between 1.0 and 1.125 -> even
    assert oracle.e4m3_encode(1.1875) == 0x3A  # tie between 1.125 and 1.25 -> even
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_decode(0x7E) == fmt["e4m3_ocp_max"]
    assert oracle.e4m3_decode(0x39) - oracle.e4m3_decode(0x38) == fmt["e4m3_spacing_above_1"]
    assert oracle.e4m3_encode(1e9) == 0x7E and oracle.e4m3_encode(-1e9) == 0xFE  # satfinite
    # every finite code decodes and re-encodes to itself
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c
    # the largest value is the OCP one, not the fnuz one
    assert max(oracle.e4m3_decode(c) for c in range(0x7F)) == 448.0 != fmt["e4m3_fnuz_max"]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([1.00390625, 1.01171875, -2.0 ** -130, 3.0e-39])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(oracle.bf16_to_float(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).double().numpy())


def _ceil_by_search(amax):
    # smallest integer e with amax / 2^e <= 448, by direct search
    e = -200
    while math.ldexp(amax, -e) > 448.0:
        e += 1
    return max(-127, min(127, e))


@pytest.mark.parametrize("seed", [0, 1])
def test_ceil_exponent_is_smallest_nonclipping(seed):
    rng = np.random.default_rng(seed)
    vals = list(np.exp(rng.uniform(-90, 90, 3000)))
    for k in range(-130, 120):
        for m in (1.0, 1.5, 1.75, 1.75 + 2.0 ** -7, 2.0 - 2.0 ** -7):
            vals.append(math.ldexp(m, k))
    vals += [2.0 ** -133, 3 * 2.0 ** -133, 448.0, 449.0, 480.0, 900.0]
    for a in vals:
        a = float(oracle.bf16_to_float(oracle.to_bf16(np.array([a])))[0])  # bf16 amax
        if a == 0.0 or not math.isfinite(a):
            continue
        e = oracle.ceil_exponent(a)
        assert e == _ceil_by_search(a), a
        if -127 < e < 127:
            assert math.ldexp(a, -e) <= 448.0 < math.ldexp(a, -(e - 1))
    assert oracle.ceil_exponent(0.0) == 0


def _quant_block(values, rule):
    x = workloads.f32_to_bf16_bits(np.array(values, dtype=np.float32)).reshape(len(values), 1, 1)
    cu = np.array([0, len(values)], dtype=np.int32)
    codes, exps = oracle.quantize(x, cu, block=32, rule=rule)
    e = int(exps[0, 0]) - 127
    return e, codes[:, 0, 0].tolist(), oracle.dequantize(codes, exps)[:, 0, 0].tolist()


def test_ceil_rule_examples(golden):
    for case in golden("quantizer_examples.json")["ceil_rule"]["cases"]:
        e, codes, rec = _quant_block(case["values"], rule=0)
        assert e == case["exponent"] and codes == case["codes"] and rec == case["reconstructed"]


def test_floor_rule_examples(golden):
    for case in golden("quantizer_examples.json")["floor_rule"]["cases"]:
        e, codes, rec = _quant_block(case["values"], rule=1)
        assert e == case["exponent"] and codes == case["codes"] and rec == case["reconstructed"]
    # the floor rule moves 480's reconstruction when 900 joins its group; the
    # ceil rule keeps it
    assert _quant_block([480.0], 1)[2][0] != _quant_block([480.0, 900.0], 1)[2][0]
    assert _quant_block([480.0], 0)[2][0] == _quant_block([480.0, 900.0], 0)[2][0]


def test_range_budget_clip(golden):
    rb = golden("quantizer_examples.json")["range_budget"]
    assert oracle.e4m3_decode(oracle.e4m3_encode(rb["boost"])) == rb["default_bound"]  # p = 1
    clipped = oracle.e4m3_decode(oracle.e4m3_encode(rb["tempting_bound"]))
    assert clipped == rb["clipped_code_value"]
    assert clipped / rb["boost"] == rb["reconstructed_weight"] != rb["intended_weight"]


def test_lattice_shift_preserves_normal_values(golden):
    rng = np.random.default_rng(3)
    y = rng.standard_normal(20000) * 100
    for v in y:
        c1 = oracle.e4m3_encode(v)
        c2 = oracle.e4m3_encode(v / 2)
        if abs(oracle.e4m3_decode(c1)) >= 2.0 ** -6 * 2 and abs(v) < 448:
            # both codes normal and unclipped: same represented value
            assert oracle.e4m3_decode(c1) == 2 * oracle.e4m3_decode(c2)
    # subnormal boundary: the smallest subnormal at scale s is a tie at 2s
    sub = golden("quantizer_examples.json")["subnormal_boundary"]["smallest_subnormal"]
    assert oracle.e4m3_decode(oracle.e4m3_encode(sub)) == sub
    assert oracle.e4m3_decode(oracle.e4m3_encode(sub / 2)) == 0.0


def test_outlier_example_loose(golden):
    g = golden("outlier_example.json")
    flush, med_t, med_b = [], [], []
    for seed in range(10):
        rng = np.random.default_rng(seed)
        small = rng.standard_normal(g["n_small"]) * g["small_size"]
        s = 448.0 / g["outlier"]
        rec = np.array([oracle.e4m3_decode(oracle.e4m3_encode(v * s)) / s for v in small])
        flush.append(np.mean(rec == 0))
        med_t.append(np.median(np.abs(rec - small) / np.abs(small)))
        errs = []
        for blk in small.reshape(-1, 128):
            sb = 448.0 / np.abs(blk).max()
            rb = np.array([oracle.e4m3_decode(oracle.e4m3_encode(v * sb)) / sb for v in blk])
            errs.append(np.abs(rb - blk) / np.abs(blk))
        med_b.append(np.median(np.concatenate(errs)))
    assert abs(np.mean(flush) - g["per_tensor_flush_frac"]) < 0.04
    assert abs(np.mean(med_t) - g["per_tensor_median_rel_err"]) < 0.04
    assert abs(np.mean(med_b) - g["block128_median_rel_err"]) < 0.01


def test_quantizer_blocks_are_document_local():
    # documents of 40 and 50 tokens starting at an unaligned offset: blocks
    # [0,32) [32,40) [40,72) [72,90); a huge value in one block changes no
    # other block's exponent
    rng = np.random.default_rng(1)
    x = rng.standard_normal((96, 2, 8)).astype(np.float32)
    cu = np.array([0, 40, 90], dtype=np.int32)
    bx = workloads.f32_to_bf16_bits(x)
    c0, e0 = oracle.quantize(bx, cu)
    x2 = x.copy()
    x2[45, 1, 3] = 1e4
    c1, e1 = oracle.quantize(workloads.f32_to_bf16_bits(x2), cu)
    changed = np.nonzero(e0[1] != e1[1])[0]
    assert changed.min() == 40 and changed.max() == 71
    assert np.array_equal(e0[0], e1[0])
    # exponents are constant on each block and follow its own amax
    for (s, t) in [(0, 32), (32, 40), (40, 72), (72, 90)]:
        for h in range(2):
            assert len(set(e0[h, s:t].tolist())) == 1
            amax = np.abs(workloads.bf16_bits_to_f32(bx[s:t, h])).max()
            assert int(e0[h, s]) - 127 == oracle.ceil_exponent(float(amax))
    # padding rows: zero codes, exponent byte 127
    assert np.all(c0[90:] == 0) and np.all(e0[:, 90:] == 127)


def test_per_token_option_is_one_block_per_token():
    rng = np.random.default_rng(2)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((70, 1, 16)).astype(np.float32))
    cu = np.array([0, 70], dtype=np.int32)
    codes, exps = oracle.quantize(x, cu, block=1)
    for t in range(70):
        amax = np.abs(workloads.bf16_bits_to_f32(x[t, 0])).max()
        assert int(exps[0, t]) - 127 == oracle.ceil_exponent(float(amax))


def _nvfp4_brute(v, s):
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    best = None
    for c, g in enumerate(grid):
        err = abs(abs(v) - g * s)
        if best is None or err < best[0] or (err == best[0] and c % 2 == 0):
            best = (err, c)
    return best[1] | (8 if math.copysign(1.0, v) < 0 else 0)


def test_nvfp4_view_matches_brute_force():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 2, 32)).astype(np.float32) * np.float32(3.0)
    x[0, 0, :16] = 0.0
    bx = workloads.f32_to_bf16_bits(x)
    xf = workloads.bf16_bits_to_f32(bx).astype(np.float64)
    cu = np.array([0, 9], dtype=np.int32)
    codes, scales = oracle.quantize_nvfp4(bx, cu)
    for t in range(9):
        for h in range(2):
            for g in range(2):
                grp = xf[t, h, 16 * g:16 * g + 16]
                s = oracle.e4m3_decode(scales[t, h, g])
                amax = np.abs(grp).max()
                if amax == 0:
                    assert s == 1.0
                else:
                    # smallest E4M3 value with amax / s <= 6
                    cands = [oracle.e4m3_decode(c) for c in range(1, 0x7F)]
                    assert s == min(c for c in cands if amax / c <= 6.0)
                for c in range(16):
                    k = 16 * g + c
                    byte = codes[t, h, k // 2]
                    code = (byte & 15) if k % 2 == 0 else (byte >> 4)
                    assert code == _nvfp4_brute(grp[c], s)
