"""ctypes binding of libflamia.so (the C ABI in include/flamia.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or a call fails, an exception
is raised."""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflamia.so")

FLAMIA_OK = 0
FLAMIA_ERR_INVALID_ARG = 1
FLAMIA_ERR_UNSUPPORTED = 2
FLAMIA_ERR_WORKSPACE = 3
FLAMIA_ERR_HIP = 4

FLAMIA_CAUSAL = 1 << 0
FLAMIA_EXACT = 1 << 1
FLAMIA_FP4_SCORE = 1 << 2
FLAMIA_DETERMINISTIC = 1 << 3
FLAMIA_HADAMARD = 1 << 4
FLAMIA_DQ_PRESCALE_SEQUENCE = 1 << 5  # test-only negative control (backward)

FLAMIA_SCALE_TOKBLOCK32 = 0
FLAMIA_SCALE_PER_TOKEN = 1
FLAMIA_SCALE_NVFP4_16 = 2
FLAMIA_SCALE_ROTATE = 0x100
FLAMIA_SCALE_FLOOR_CONTROL = 0x200

EXPORTED = [
    "flamia_quantize_tokblock",
    "flamia_quantize_qkv",
    "flamia_attn_fwd_workspace_size",
    "flamia_attn_fwd",
    "flamia_attn_fwd_noalloc_scratch_bytes",
    "flamia_attn_fwd_noalloc",
    "flamia_attn_bwd_workspace_size",
    "flamia_attn_bwd",
    "flamia_attn_bwd_workspace_layout",
    "flamia_status_string",
]


class FlamiaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))


class flamia_kernel_events(ctypes.Structure):
    _fields_ = [("attn_start", ctypes.c_void_p), ("attn_stop", ctypes.c_void_p)]


class flamia_problem(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("events", ctypes.POINTER(flamia_kernel_events)),
    ]


class flamia_bwd_workspace_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("do_codes", "do_exps", "delta", "dq_prescale", "dq_accum", "total")]


_lib = None


def load():
    """Load libflamia.so (built by bit_causal_flash_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libflamia.so is not built: run `python -m bit_causal_flash_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(flamia_problem)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.flamia_quantize_tokblock.restype = ctypes.c_int
    lib.flamia_quantize_tokblock.argtypes = [P, i32, i32, vp, vp, vp, vp]
    lib.flamia_quantize_qkv.restype = ctypes.c_int
    lib.flamia_quantize_qkv.argtypes = [P, i32] + [vp] * 10
    lib.flamia_attn_fwd_workspace_size.restype = sz
    lib.flamia_attn_fwd_workspace_size.argtypes = [P]
    lib.flamia_attn_fwd.restype = ctypes.c_int
    lib.flamia_attn_fwd.argtypes = [P] + [vp] * 12 + [vp, sz, vp]
    lib.flamia_attn_fwd_noalloc_scratch_bytes.restype = sz
    lib.flamia_attn_fwd_noalloc_scratch_bytes.argtypes = []
    lib.flamia_attn_fwd_noalloc.restype = ctypes.c_int
    lib.flamia_attn_fwd_noalloc.argtypes = [P] + [vp] * 12 + [vp]
    lib.flamia_attn_bwd_workspace_size.restype = sz
    lib.flamia_attn_bwd_workspace_size.argtypes = [P]
    lib.flamia_attn_bwd.restype = ctypes.c_int
    lib.flamia_attn_bwd.argtypes = [P] + [vp] * 16 + [vp, sz, vp]
    lib.flamia_attn_bwd_workspace_layout.restype = ctypes.c_int
    lib.flamia_attn_bwd_workspace_layout.argtypes = [P, ctypes.POINTER(flamia_bwd_workspace_layout)]
    lib.flamia_status_string.restype = ctypes.c_char_p
    lib.flamia_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().flamia_status_string(int(status)).decode()


def _check(fn, status):
    if status != FLAMIA_OK:
        raise FlamiaError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_problem(cu_seqlens, total_tokens: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, softmax_scale: float = 0.0, flags: int = FLAMIA_CAUSAL):
    """cu_seqlens: device int32 tensor [B + 1] (kept alive by the problem)."""
    p = flamia_problem(int(total_tokens), int(cu_seqlens.numel()) - 1,
                       ctypes.c_void_p(cu_seqlens.data_ptr()), int(num_q_heads),
                       int(num_kv_heads), int(head_dim), float(softmax_scale), int(flags), None)
    p._cu = cu_seqlens
    return p


def set_events(p, start, stop):
    """Make the next attention calls with `p` record hipEvent_t handles
    `start` / `stop` (ints) around their main kernel; None clears them."""
    if start is None and stop is None:
        p.events = None
        p._ev = None
        return
    ev = flamia_kernel_events(ctypes.c_void_p(start), ctypes.c_void_p(stop))
    p._ev = ev
    p.events = ctypes.pointer(ev)


def softmax_scale_of(p) -> float:
    return p.softmax_scale if p.softmax_scale > 0 else 1.0 / math.sqrt(p.head_dim)


def flamia_quantize_tokblock(p, num_heads, scale_mode, x, codes, exps, stream=None):
    _check("flamia_quantize_tokblock",
           load().flamia_quantize_tokblock(ctypes.byref(p), int(num_heads), int(scale_mode),
                                           _ptr(x), _ptr(codes), _ptr(exps), _stream(stream)))


def flamia_quantize_qkv(p, scale_mode, q, k, v, q_codes, q_exps, k_codes, k_exps, v_codes, v_exps,
                        stream=None):
    _check("flamia_quantize_qkv",
           load().flamia_quantize_qkv(ctypes.byref(p), int(scale_mode), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(q_codes), _ptr(q_exps), _ptr(k_codes), _ptr(k_exps),
                                      _ptr(v_codes), _ptr(v_exps), _stream(stream)))


def flamia_attn_fwd_workspace_size(p) -> int:
    return int(load().flamia_attn_fwd_workspace_size(ctypes.byref(p)))


def flamia_attn_bwd_workspace_size(p) -> int:
    return int(load().flamia_attn_bwd_workspace_size(ctypes.byref(p)))


def flamia_attn_bwd_workspace_layout(p) -> flamia_bwd_workspace_layout:
    out = flamia_bwd_workspace_layout()
    _check("flamia_attn_bwd_workspace_layout",
           load().flamia_attn_bwd_workspace_layout(ctypes.byref(p), ctypes.byref(out)))
    return out


def flamia_attn_fwd(p, q_codes, q_exps, k_codes, k_exps, v_codes, v_exps, o, lse, workspace,
                    fp4=None, stream=None):
    q4, q4s, k4, k4s = fp4 if fp4 is not None else (None, None, None, None)
    _check("flamia_attn_fwd", load().flamia_attn_fwd(
        ctypes.byref(p), _ptr(q_codes), _ptr(q_exps), _ptr(k_codes), _ptr(k_exps), _ptr(v_codes),
        _ptr(v_exps), _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(o), _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def flamia_attn_fwd_noalloc(p, q_codes, q_exps, k_codes, k_exps, v_codes, v_exps, o, lse,
                            fp4=None, stream=None):
    q4, q4s, k4, k4s = fp4 if fp4 is not None else (None, None, None, None)
    _check("flamia_attn_fwd_noalloc", load().flamia_attn_fwd_noalloc(
        ctypes.byref(p), _ptr(q_codes), _ptr(q_exps), _ptr(k_codes), _ptr(k_exps), _ptr(v_codes),
        _ptr(v_exps), _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(o), _ptr(lse),
        _stream(stream)))


def flamia_attn_noalloc_scratch_bytes() -> int:
    return int(load().flamia_attn_fwd_noalloc_scratch_bytes())


def flamia_attn_bwd(p, q_codes, q_exps, k_codes, k_exps, v_codes, v_exps, o, lse, dout, dq, dk,
                    dv, workspace, fp4=None, stream=None):
    q4, q4s, k4, k4s = fp4 if fp4 is not None else (None, None, None, None)
    _check("flamia_attn_bwd", load().flamia_attn_bwd(
        ctypes.byref(p), _ptr(q_codes), _ptr(q_exps), _ptr(k_codes), _ptr(k_exps), _ptr(v_codes),
        _ptr(v_exps), _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(o), _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


# ---------------------------------------------------------------------------
# torch-facing conveniences (allocation only)
# ---------------------------------------------------------------------------

def quantize(p, x, num_heads, scale_mode=FLAMIA_SCALE_TOKBLOCK32, stream=None):
    """x: bf16 (or int16 bit patterns) [T][H][d] on the GPU -> (codes uint8, exps uint8)."""
    import torch
    T, H, d = x.shape
    codes = torch.empty((T, H, d), dtype=torch.uint8, device=x.device)
    exps = torch.empty((H, T), dtype=torch.uint8, device=x.device)
    flamia_quantize_tokblock(p, num_heads, scale_mode, x, codes, exps, stream)
    return codes, exps


def quantize_qkv(p, q, k, v, scale_mode=FLAMIA_SCALE_TOKBLOCK32, stream=None):
    """Q, K, V in one launch -> ((q codes, q exps), (k ...), (v ...))."""
    import torch
    out = []
    for x in (q, k, v):
        T, H, d = x.shape
        out.append((torch.empty((T, H, d), dtype=torch.uint8, device=x.device),
                    torch.empty((H, T), dtype=torch.uint8, device=x.device)))
    flamia_quantize_qkv(p, scale_mode, q, k, v, out[0][0], out[0][1], out[1][0], out[1][1],
                        out[2][0], out[2][1], stream)
    return tuple(out)


def quantize_nvfp4(p, x, num_heads, stream=None):
    """x: bf16 [T][H][d] -> E2M1 score view (codes uint8 [T][H][d/2], E4M3
    scales uint8 [T][H][d/16])."""
    import torch
    T, H, d = x.shape
    codes = torch.empty((T, H, d // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((T, H, d // 16), dtype=torch.uint8, device=x.device)
    flamia_quantize_tokblock(p, num_heads, FLAMIA_SCALE_NVFP4_16, x, codes, scales, stream)
    return codes, scales


def attn_fwd(p, q, k, v, stream=None, fp4=None):
    """q, k, v: (codes, exps) pairs; fp4: optional ((q codes, q scales),
    (k codes, k scales)) E2M1 score views.  Returns (o bf16 [T][Hq][d],
    lse [Hq][T])."""
    import torch
    dev = q[0].device
    T, Hq, d = q[0].shape
    o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty(max(flamia_attn_fwd_workspace_size(p), 1), dtype=torch.uint8, device=dev)
    f4 = None if fp4 is None else (fp4[0][0], fp4[0][1], fp4[1][0], fp4[1][1])
    flamia_attn_fwd(p, q[0], q[1], k[0], k[1], v[0], v[1], o, lse, ws, fp4=f4, stream=stream)
    if stream is not None:
        # the workspace was allocated on the current stream but is used on
        # `stream`: keep the caching allocator from reusing it before that
        # stream's kernels are done
        ws.record_stream(stream)
    return o, lse


def attn_bwd(p, q, k, v, o, lse, dout, stream=None, workspace=None, fp4=None):
    """Returns (dq, dk, dv, workspace)."""
    import torch
    dev = q[0].device
    T, Hq, d = q[0].shape
    Hkv = k[0].shape[1]
    dq = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=dev)
    dk = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev)
    dv = torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.empty(max(flamia_attn_bwd_workspace_size(p), 1), dtype=torch.uint8,
                                device=dev)
    f4 = None if fp4 is None else (fp4[0][0], fp4[0][1], fp4[1][0], fp4[1][1])
    flamia_attn_bwd(p, q[0], q[1], k[0], k[1], v[0], v[1], o, lse, dout, dq, dk, dv, workspace,
                    fp4=f4, stream=stream)
    if stream is not None:
        workspace.record_stream(stream)
    return dq, dk, dv, workspace


# ---------------------------------------------------------------------------
# PyTorch operator: quantize + forward, and the backward, as one autograd
# Function (FLAMIA review section 9 "Reproduction notes and limitations": the
# method ships as graph-capturable PyTorch operators taking bf16 in and
# returning bf16 out).  torch supplies memory and the current stream only.
# ---------------------------------------------------------------------------

_ATTN_FN = None


def _attn_function():
    global _ATTN_FN
    if _ATTN_FN is not None:
        return _ATTN_FN
    import torch

    class FlamiaAttn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, cu_seqlens, flags, softmax_scale):
            T, Hq, d = q.shape
            Hkv = k.shape[1]
            p = make_problem(cu_seqlens, T, Hq, Hkv, d, softmax_scale, flags)
            mode = FLAMIA_SCALE_PER_TOKEN if flags & FLAMIA_EXACT else FLAMIA_SCALE_TOKBLOCK32
            if flags & FLAMIA_HADAMARD:
                mode |= FLAMIA_SCALE_ROTATE  # Q and K only (flamia_quantize_qkv)
            (qc, qe), (kc, ke), (vc, ve) = quantize_qkv(p, q, k, v, mode)
            views = ()
            if flags & FLAMIA_FP4_SCORE:
                views = quantize_nvfp4(p, q, Hq) + quantize_nvfp4(p, k, Hkv)
            fp4 = None if not views else ((views[0], views[1]), (views[2], views[3]))
            o, lse = attn_fwd(p, (qc, qe), (kc, ke), (vc, ve), fp4=fp4)
            ctx.save_for_backward(cu_seqlens, qc, qe, kc, ke, vc, ve, o, lse, *views)
            ctx.flags = flags
            ctx.scale = softmax_scale
            ctx.mark_non_differentiable(lse)
            return o, lse

        @staticmethod
        def backward(ctx, dout, _dlse):
            cu, qc, qe, kc, ke, vc, ve, o, lse, *views = ctx.saved_tensors
            T, Hq, d = qc.shape
            p = make_problem(cu, T, Hq, kc.shape[1], d, ctx.scale, ctx.flags)
            fp4 = None if not views else ((views[0], views[1]), (views[2], views[3]))
            dout = dout.to(torch.bfloat16).contiguous()
            dq, dk, dv, _ = attn_bwd(p, (qc, qe), (kc, ke), (vc, ve), o, lse, dout, fp4=fp4)
            return dq, dk, dv, None, None, None

    _ATTN_FN = FlamiaAttn
    return FlamiaAttn


def attn(q, k, v, cu_seqlens, causal=True, exact=False, fp4_score=False, hadamard=False,
         deterministic=False, softmax_scale=0.0, return_lse=False):
    """Causal packed microscaled attention as a differentiable operator.

    q: bf16 [T][Hq][d], k, v: bf16 [T][Hkv][d] (packed documents, rows past
    cu_seqlens[-1] are padding), cu_seqlens: int32 [B + 1] on the same device.
    The forward quantizes Q, K, V (token blocks, or per token with `exact`;
    the E2M1 score views with `fp4_score`; Q and K rotated with `hadamard`)
    and runs flamia_attn_fwd; the backward runs flamia_attn_bwd, which
    quantizes dO itself.  Returns O (bf16 [T][Hq][d]), and with `return_lse`
    also the natural-log LSE (float32 [Hq][T], not differentiable).  Raises
    if the library is missing or the inputs are not bf16 GPU tensors: there
    is no fallback path."""
    import torch
    for name, x in (("q", q), ("k", k), ("v", v)):
        if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 3:
            raise ValueError("%s must be a 3-d bfloat16 GPU tensor [T][H][d]" % name)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be int32 on the device of q")
    flags = (FLAMIA_CAUSAL if causal else 0) | (FLAMIA_EXACT if exact else 0) | \
        (FLAMIA_FP4_SCORE if fp4_score else 0) | (FLAMIA_HADAMARD if hadamard else 0) | \
        (FLAMIA_DETERMINISTIC if deterministic else 0)
    load()
    o, lse = _attn_function().apply(q.contiguous(), k.contiguous(), v.contiguous(),
                                    cu_seqlens.contiguous(), flags, float(softmax_scale))
    return (o, lse) if return_lse else o
