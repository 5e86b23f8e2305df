"""The allocation-free forward, flamia_attn_fwd_noalloc, through the C ABI:
two calls in a row (the second on a smaller problem, with the scratch still
holding the first call's work list) give O and LSE bit-identical to
flamia_attn_fwd with a workspace on the same inputs, and a problem whose
work list exceeds the fixed scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest

import workloads
from tests.gpu_helpers import dev, host, log

pytestmark = pytest.mark.gpu

CASES = [
    # name, lens, capacity, Hq, Hkv, d, causal
    ("larger", [700, 1, 1300, 513, 0, 420], 3000, 4, 2, 128, True),
    ("smaller", [90, 257, 33], 400, 2, 1, 64, False),
]


def _quantized(F, w, flags):
    p = F.make_problem(dev(w.cu.astype(np.int32)), w.T, w.Hq, w.Hkv, w.d, 0.0, flags)
    x = [dev(getattr(w, n).view(np.int16)) for n in ("q", "k", "v")]
    return p, F.quantize_qkv(p, *x)


def test_noalloc_forward_matches_the_workspace_forward_twice():
    import torch
    from bit_causal_flash_amd import flamia as F
    runs = []
    for name, lens, cap, Hq, Hkv, d, causal in CASES:
        w = workloads.make(name, 21, cap, lens, Hq, Hkv, d,
                           flags=workloads.FLAG_CAUSAL if causal else 0)
        p, (q, k, v) = _quantized(F, w, F.FLAMIA_CAUSAL if causal else 0)
        o = torch.full((w.T, Hq, d), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        lse = torch.full((Hq, w.T), 7.0, dtype=torch.float32, device="cuda")
        log("case %s: no-alloc forward T=%d Hq=%d d=%d causal=%d" % (name, w.T, Hq, d, causal))
        F.flamia_attn_fwd_noalloc(p, q[0], q[1], k[0], k[1], v[0], v[1], o, lse)
        runs.append((p, q, k, v, o, lse))
    torch.cuda.synchronize()
    for (name, *_), (p, q, k, v, o, lse) in zip(CASES, runs):
        o_ref, lse_ref = F.attn_fwd(p, q, k, v)
        torch.cuda.synchronize()
        assert np.array_equal(host(o), host(o_ref)), name + " O"
        assert np.array_equal(host(lse), host(lse_ref)), name + " LSE"
        log("case %s: bit-identical to the workspace forward" % name)


def test_noalloc_forward_refuses_a_problem_beyond_its_scratch():
    from bit_causal_flash_amd import flamia as F
    lib = F.load()
    cap = F.flamia_attn_noalloc_scratch_bytes()
    assert cap == 4 << 20
    vp = ctypes.c_void_p(16)  # never dereferenced: the call returns before any launch
    big = F.flamia_problem(1 << 21, 1 << 20, vp, 1, 1, 64, 0.0, F.FLAMIA_CAUSAL, None)
    assert F.flamia_attn_fwd_workspace_size(big) > cap
    st = lib.flamia_attn_fwd_noalloc(ctypes.byref(big), *([vp] * 6), None, None, None, None, vp,
                                     vp, None)
    assert st == F.FLAMIA_ERR_WORKSPACE
    ok = F.flamia_problem(1 << 18, 1 << 18, vp, 1, 1, 64, 0.0, F.FLAMIA_CAUSAL, None)
    assert F.flamia_attn_fwd_workspace_size(ok) <= cap
