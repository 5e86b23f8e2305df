"""The C ABI on the CPU: the library loads, exports every declared entry
point, and rejects bad host-side arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from bit_causal_flash_amd import flamia as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "flamia.h")).read()
    names = re.findall(r"^[A-Za-z_ *]*?\b(flamia_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declarations_are_exported():
    lib = F.load()
    names = declared_functions()
    assert set(F.EXPORTED) == set(names)
    for n in names:
        assert hasattr(lib, n), n


def _problem(T=64, B=1, Hq=2, Hkv=1, d=128, flags=F.FLAMIA_CAUSAL, cu=8):
    return F.flamia_problem(T, B, ctypes.c_void_p(cu), Hq, Hkv, d, 0.0, flags, None)


def test_invalid_arguments_rejected_before_launch():
    lib = F.load()
    vp = ctypes.c_void_p(16)
    P = ctypes.byref
    assert lib.flamia_quantize_tokblock(None, 1, 0, vp, vp, vp, None) == F.FLAMIA_ERR_INVALID_ARG
    assert lib.flamia_quantize_tokblock(P(_problem(d=96)), 1, 0, vp, vp, vp, None) == \
        F.FLAMIA_ERR_UNSUPPORTED
    assert lib.flamia_quantize_tokblock(P(_problem(d=0)), 1, 0, vp, vp, vp, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    assert lib.flamia_quantize_tokblock(P(_problem()), 0, 0, vp, vp, vp, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    assert lib.flamia_quantize_tokblock(P(_problem()), 1, 7, vp, vp, vp, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    assert lib.flamia_quantize_tokblock(P(_problem()), 1, 0, None, vp, vp, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    assert lib.flamia_quantize_tokblock(P(_problem(B=0)), 1, 0, vp, vp, vp, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    assert lib.flamia_quantize_tokblock(P(_problem(T=-1)), 1, 0, vp, vp, vp, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    assert lib.flamia_quantize_tokblock(P(_problem(cu=0)), 1, 0, vp, vp, vp, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    # empty input is a no-op
    assert lib.flamia_quantize_tokblock(P(_problem(T=0)), 1, 0, None, None, None, None) == F.FLAMIA_OK

    args12 = [vp] * 6 + [None] * 4 + [vp, vp]
    ws = F.flamia_attn_fwd_workspace_size(_problem())
    assert ws > 0
    fwd = lib.flamia_attn_fwd
    assert fwd(P(_problem(Hq=3, Hkv=2)), *args12, vp, ws, None) == F.FLAMIA_ERR_INVALID_ARG
    assert fwd(P(_problem(flags=1 << 7)), *args12, vp, ws, None) == F.FLAMIA_ERR_INVALID_ARG
    assert fwd(P(_problem(flags=F.FLAMIA_FP4_SCORE)), *args12, vp, ws, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    assert fwd(P(_problem()), *args12, vp, ws - 1, None) == F.FLAMIA_ERR_WORKSPACE
    assert fwd(P(_problem()), *args12, None, ws, None) == F.FLAMIA_ERR_WORKSPACE
    bad_fp4 = [vp] * 6 + [vp, None, None, None] + [vp, vp]
    assert fwd(P(_problem()), *bad_fp4, vp, ws, None) == F.FLAMIA_ERR_INVALID_ARG
    # the E2M1 score views are required with FP4_SCORE, which requires EXACT
    fp4_flags = F.FLAMIA_CAUSAL | F.FLAMIA_EXACT | F.FLAMIA_FP4_SCORE
    assert fwd(P(_problem(flags=fp4_flags)), *args12, vp, ws, None) == F.FLAMIA_ERR_INVALID_ARG
    assert fwd(P(_problem(flags=fp4_flags)), *bad_fp4, vp, ws, None) == F.FLAMIA_ERR_INVALID_ARG
    assert fwd(P(_problem(T=0)), *([None] * 12), None, 0, None) == F.FLAMIA_OK

    wsb = F.flamia_attn_bwd_workspace_size(_problem())
    args16 = [vp] * 6 + [None] * 4 + [vp] * 6
    bwd = lib.flamia_attn_bwd
    assert bwd(P(_problem()), *args16, vp, wsb - 1, None) == F.FLAMIA_ERR_WORKSPACE
    assert bwd(P(_problem(Hkv=0)), *args16, vp, wsb, None) == F.FLAMIA_ERR_INVALID_ARG
    missing = [vp] * 6 + [None] * 4 + [vp, vp, vp, None, vp, vp]
    assert bwd(P(_problem()), *missing, vp, wsb, None) == F.FLAMIA_ERR_INVALID_ARG
    # the exact-scale backward has no deterministic dQ pass, and its E2M1
    # score path covers head_dim 64 only
    det_exact = F.FLAMIA_CAUSAL | F.FLAMIA_EXACT | F.FLAMIA_DETERMINISTIC
    assert bwd(P(_problem(flags=det_exact)), *args16, vp, wsb, None) == F.FLAMIA_ERR_UNSUPPORTED
    # the Hadamard option: not with the exact-scale option, and no
    # deterministic backward; the rotation bit only with the E4M3 policies
    had = F.FLAMIA_CAUSAL | F.FLAMIA_HADAMARD
    assert fwd(P(_problem(flags=had | F.FLAMIA_EXACT)), *args12, vp, ws, None) == \
        F.FLAMIA_ERR_UNSUPPORTED
    assert bwd(P(_problem(flags=had | F.FLAMIA_DETERMINISTIC)), *args16, vp, wsb, None) == \
        F.FLAMIA_ERR_UNSUPPORTED
    # the sequence-wide prescale control has no deterministic backward (FP32
    # dQ, no prescale); bit 5 is a known flag, bit 7 is not
    seqc = F.FLAMIA_CAUSAL | F.FLAMIA_DQ_PRESCALE_SEQUENCE
    assert bwd(P(_problem(flags=seqc | F.FLAMIA_DETERMINISTIC)), *args16, vp, wsb, None) == \
        F.FLAMIA_ERR_UNSUPPORTED
    assert F.flamia_attn_bwd_workspace_size(_problem(flags=seqc)) == wsb
    q = lib.flamia_quantize_tokblock
    assert q(P(_problem()), 1, F.FLAMIA_SCALE_NVFP4_16 | F.FLAMIA_SCALE_ROTATE, vp, vp, vp, None) == \
        F.FLAMIA_ERR_INVALID_ARG
    assert q(P(_problem()), 1, 5 | F.FLAMIA_SCALE_ROTATE, vp, vp, vp, None) == F.FLAMIA_ERR_INVALID_ARG
    assert q(P(_problem(T=0)), 1, F.FLAMIA_SCALE_ROTATE, None, None, None, None) == F.FLAMIA_OK
    assert q(P(_problem()), 1, F.FLAMIA_SCALE_NVFP4_16 | F.FLAMIA_SCALE_FLOOR_CONTROL, vp, vp, vp,
             None) == F.FLAMIA_ERR_INVALID_ARG
    qkv = lib.flamia_quantize_qkv
    nine = [vp] * 9  # q, k, v, then codes and exponents of each
    assert qkv(P(_problem()), F.FLAMIA_SCALE_NVFP4_16, *nine, None) == F.FLAMIA_ERR_INVALID_ARG
    assert qkv(P(_problem()), 0, *([vp] * 8), None, None) == F.FLAMIA_ERR_INVALID_ARG
    assert qkv(P(_problem(d=96)), 0, *nine, None) == F.FLAMIA_ERR_UNSUPPORTED
    assert qkv(P(_problem(T=0)), 0, *([None] * 9), None) == F.FLAMIA_OK
    with4 = [vp] * 16
    assert bwd(P(_problem(d=128, flags=fp4_flags)), *with4, vp,
               F.flamia_attn_bwd_workspace_size(_problem(d=128, flags=fp4_flags)), None) == \
        F.FLAMIA_ERR_UNSUPPORTED


def test_workspace_layout_is_consistent():
    p = _problem(T=1000, B=3, Hq=8, Hkv=2, d=64)
    L = F.flamia_attn_bwd_workspace_layout(p)
    T, Hq, d = 1000, 8, 64
    assert L.do_codes == 0 and L.do_exps >= T * Hq * d
    assert L.delta >= L.do_exps + Hq * T and L.dq_prescale >= L.delta + 4 * Hq * T
    assert L.dq_accum >= L.dq_prescale + Hq * T
    assert L.total >= L.dq_accum + 2 * T * Hq * d
    assert L.total == F.flamia_attn_bwd_workspace_size(p)
    for off in (L.do_exps, L.delta, L.dq_prescale, L.dq_accum):
        assert off % 256 == 0


def test_status_strings():
    for s in range(5):
        assert F.status_string(s)
