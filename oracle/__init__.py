"""FP64 CPU oracle for causal packed microscaled attention (the FLAMIA method).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The HIP product
path never imports, links or calls it, and the two share no code.

This module is argument marshalling around ``flamia_oracle.c`` (numpy arrays
in, numpy arrays out); the arithmetic lives in the C file, whose header lists
the pages and sections each routine follows.

Array conventions (all C-contiguous):
  bf16 tensors       uint16 [T][H][d] (raw bfloat16 bit patterns)
  E4M3 codes         uint8  [T][H][d]
  exponent tables    uint8  [H][T]   (UE8M0: e + 127, replicated per token)
  cu_seqlens         int32  [B + 1]
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flamia_oracle.c")
_LIB = os.path.join(_HERE, "_liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-fopenmp", "-fPIC", "-shared",
             "-Wall", "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
        _lib.orc_e4m3_encode.restype = ctypes.c_uint8
        _lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
        _lib.orc_e4m3_decode.restype = ctypes.c_double
        _lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        _lib.orc_bf16_to_f64.restype = ctypes.c_double
        _lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        _lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        _lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        _lib.orc_ceil_exponent.restype = ctypes.c_int
        _lib.orc_ceil_exponent.argtypes = [ctypes.c_double]
        _lib.orc_floor_exponent.restype = ctypes.c_int
        _lib.orc_floor_exponent.argtypes = [ctypes.c_double]
        _lib.orc_f16_round.restype = ctypes.c_double
        _lib.orc_f16_round.argtypes = [ctypes.c_double]
        _lib.orc_bwd_dq_ranges.restype = ctypes.c_int64
        _lib.orc_bwd_dkdv_ranges.restype = ctypes.c_int64
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _check(rc):
    if rc != 0:
        raise OracleError("oracle returned %d" % rc)


# --------------------------------------------------------------------------
# scalar format helpers
# --------------------------------------------------------------------------

def e4m3_encode(y: float) -> int:
    return int(_load().orc_e4m3_encode(float(y)))


def e4m3_decode(c: int) -> float:
    return float(_load().orc_e4m3_decode(int(c)))


def bf16_to_f64(h: int) -> float:
    return float(_load().orc_bf16_to_f64(int(h)))


def f64_to_bf16(x: float) -> int:
    return int(_load().orc_f64_to_bf16(float(x)))


def ceil_exponent(amax: float) -> int:
    return int(_load().orc_ceil_exponent(float(amax)))


def floor_exponent(amax: float) -> int:
    return int(_load().orc_floor_exponent(float(amax)))


def f16_round(x: float) -> float:
    """Nearest IEEE binary16 value (ties to even), as a float."""
    return _load().orc_f16_round(float(x))


def to_bf16(x) -> np.ndarray:
    """FP64 array -> bf16 bit patterns (nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f64_to_bf16_array(ctypes.c_int64(x.size), _p(x), _p(out))
    return out


def bf16_to_float(h) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().orc_num_threads())


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------

def quantize(x, cu, block: int = 32, rule: int = 0):
    """Token-block E4M3 quantizer.  x bf16 [T][H][d] -> (codes [T][H][d],
    exps [H][T]).  block 32 = default policy, 1 = per-token option;
    rule 0 = conservative ceil exponent, 1 = floor exponent (control)."""
    x = _c(x, np.uint16)
    cu = _c(cu, np.int32)
    T, H, d = x.shape
    codes = np.empty((T, H, d), dtype=np.uint8)
    exps = np.empty((H, T), dtype=np.uint8)
    _check(_load().orc_quantize(T, len(cu) - 1, _p(cu), H, d, _p(x), block, rule,
                                _p(codes), _p(exps)))
    return codes, exps


def hadamard_matrix(d: int):
    """Sylvester Hadamard matrix H_d (float64 [d][d]): entry (i, j) is
    (-1)^popcount(i & j); H_d is symmetric and H_d H_d = d I."""
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def hadamard_rotate(x):
    """Rows of bf16 x [T][H][d] times H_d, by the FP32 fast Walsh-Hadamard
    transform (stages h = 1, 2, ..., d/2) -> float32 [T][H][d]."""
    x = _c(x, np.uint16)
    T, H, d = x.shape
    out = np.empty((T, H, d), dtype=np.float32)
    _check(_load().orc_hadamard_rotate(T, H, d, _p(x), _p(out)))
    return out


def quantize_f32(x, cu, block: int = 32, rule: int = 0):
    """The token-block quantizer over FP32 values [T][H][d]."""
    x = _c(x, np.float32)
    cu = _c(cu, np.int32)
    T, H, d = x.shape
    codes = np.empty((T, H, d), dtype=np.uint8)
    exps = np.empty((H, T), dtype=np.uint8)
    _check(_load().orc_quantize_f32(T, len(cu) - 1, _p(cu), H, d, _p(x), block, rule,
                                    _p(codes), _p(exps)))
    return codes, exps


def quantize_rotated(x, cu, block: int = 32):
    """Score-path operand with the Hadamard rotation: the rows of bf16 x
    rotated (hadamard_rotate), then quantized by the token-block rule."""
    return quantize_f32(hadamard_rotate(x), cu, block=block)


def unrotate(g):
    """Gradient with respect to a rotated operand (x_r = x H_d) taken back to
    the original coordinates: dL/dx = dL/dx_r H_d, for every row of float64
    g [T][H][d].  The rotated problem runs at softmax scale / d, since
    q_r . k_r = d q . k."""
    g = np.asarray(g, dtype=np.float64)
    return g @ hadamard_matrix(g.shape[-1])


def quantize_nvfp4(x, cu):
    """E2M1 + E4M3-per-16 score view.  -> (codes [T][H][d/2], scales
    [T][H][d/16])."""
    x = _c(x, np.uint16)
    cu = _c(cu, np.int32)
    T, H, d = x.shape
    codes = np.empty((T, H, d // 2), dtype=np.uint8)
    scales = np.empty((T, H, d // 16), dtype=np.uint8)
    _check(_load().orc_quantize_nvfp4(T, len(cu) - 1, _p(cu), H, d, _p(x), _p(codes),
                                      _p(scales)))
    return codes, scales


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

MODE_ROUNDED = 0      # microscaled forward, l = sum of rounded weights
MODE_UNROUNDED = 1    # microscaled forward, l = sum of unrounded weights
MODE_REFERENCE = 2    # FP64 online softmax without probability rounding
MODE_TILED = 3        # microscaled forward in the tile loop (running reference)


def dequantize(codes, exps):
    """E4M3 codes [T][H][d] and exponent table [H][T] -> float64 [T][H][d]."""
    codes = _c(codes, np.uint8)
    exps = _c(exps, np.uint8)
    T, H, d = codes.shape
    out = np.empty((T, H, d), dtype=np.float64)
    _load().orc_dequantize(T, H, d, _p(codes), _p(exps), _p(out))
    return out


def dequantize_nvfp4(codes, scales):
    """E2M1 codes [T][H][d/2] and E4M3 scales [T][H][d/16] -> float64."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    T, H, half = codes.shape
    out = np.empty((T, H, 2 * half), dtype=np.float64)
    _load().orc_dequantize_nvfp4(T, H, 2 * half, _p(codes), _p(scales), _p(out))
    return out


class Operands:
    """Dequantized Q, K, V (float64 [T][H][d]) of one problem, plus an
    optional separate score view of Q and K (the E2M1 route)."""

    def __init__(self, Q, K, V, Qs=None, Ks=None):
        self.Q = _c(Q, np.float64)
        self.K = _c(K, np.float64)
        self.V = _c(V, np.float64)
        self.Qs = _c(Qs, np.float64)
        self.Ks = _c(Ks, np.float64)

    @classmethod
    def from_codes(cls, q, k, v, q4=None, k4=None):
        """q, k, v: (codes, exps) pairs; q4, k4: optional (codes, scales)."""
        return cls(dequantize(*q), dequantize(*k), dequantize(*v),
                   None if q4 is None else dequantize_nvfp4(*q4),
                   None if k4 is None else dequantize_nvfp4(*k4))

    @property
    def T(self):
        return self.Q.shape[0]

    @property
    def Hq(self):
        return self.Q.shape[1]

    @property
    def Hkv(self):
        return self.K.shape[1]

    @property
    def d(self):
        return self.Q.shape[2]

    def ptrs(self):
        return [_p(self.Q), _p(self.K), _p(self.V), _p(self.Qs), _p(self.Ks)]


def attn_fwd(cu, ops: Operands, scale=None, causal=True, mode=MODE_ROUNDED, kblock=32,
             rows=None, want_rescale=False):
    """Forward.  rows: None (all) or int array [n][2] of (q head, token).
    Returns (O float64 [T][Hq][d], LSE float64 [Hq][T][, n_rescale])."""
    cu = _c(cu, np.int32)
    T, Hq, Hkv, d = ops.T, ops.Hq, ops.Hkv, ops.d
    scale = default_scale(d) if scale is None else scale
    O = np.zeros((T, Hq, d), dtype=np.float64)
    LSE = np.zeros((Hq, T), dtype=np.float64)
    nres = np.zeros((Hq, T), dtype=np.int32) if want_rescale else None
    r = None if rows is None else _c(rows, np.int32).reshape(-1, 2)
    n = 0 if r is None else r.shape[0]
    _check(_load().orc_attn_fwd(
        T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale), int(bool(causal)),
        *ops.ptrs(), mode, kblock, ctypes.c_int64(n), _p(r), _p(O), _p(LSE), _p(nres)))
    return (O, LSE, nres) if want_rescale else (O, LSE)


# --------------------------------------------------------------------------
# evaluation-noise bookkeeping (for comparisons with an FP32 implementation;
# not part of the method's arithmetic)
# --------------------------------------------------------------------------

def fwd_ties(cu, ops: Operands, noise, scale=None, causal=True, mode=MODE_TILED, kblock=64,
             rows=None):
    """Per row (float64 [Hq][T][2]): bounds on how far different roundings of
    weights lying within `noise` (fraction of each score's sum of absolute
    terms) of an E4M3 midpoint can move O (any element) and l (relative)."""
    cu = _c(cu, np.int32)
    T, Hq, Hkv, d = ops.T, ops.Hq, ops.Hkv, ops.d
    scale = default_scale(d) if scale is None else scale
    ties = np.zeros((Hq, T, 2), dtype=np.float64)
    r = None if rows is None else _c(rows, np.int32).reshape(-1, 2)
    n = 0 if r is None else r.shape[0]
    _check(_load().orc_fwd_ties(
        T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale), int(bool(causal)),
        *ops.ptrs(), mode, kblock, ctypes.c_double(noise), ctypes.c_int64(n), _p(r), _p(ties)))
    return ties


def dq_ranges(cu, ops: Operands, G, D, LSE, h, q0, noise, scale=None, causal=True,
              per_row_ds=False):
    """Near-midpoint elements of the dQ product's dS^ for the 32 rows of the
    block at q0 (head h): arrays (i, j, lo, hi), lo / hi the lowest / highest
    dS^ an evaluation within `noise` could give, minus the oracle's choice."""
    cu = _c(cu, np.int32)
    G, D, LSE = (_c(x, np.float64) for x in (G, D, LSE))
    T, Hq, Hkv, d = ops.T, ops.Hq, ops.Hkv, ops.d
    scale = default_scale(d) if scale is None else scale
    args = [T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale), int(bool(causal)),
            *ops.ptrs(), _p(G), _p(D), _p(LSE), int(bool(per_row_ds)), ctypes.c_double(noise),
            int(h), int(q0)]
    cap = 4096
    while True:
        oi, oj = np.zeros(cap, np.int32), np.zeros(cap, np.int32)
        lo, hi = np.zeros(cap), np.zeros(cap)
        n = _load().orc_bwd_dq_ranges(*args, ctypes.c_int64(cap), _p(oi), _p(oj), _p(lo), _p(hi))
        if n < 0:
            raise OracleError("oracle returned %d" % n)
        if n <= cap:
            return oi[:n], oj[:n], lo[:n], hi[:n]
        cap = int(n)


def dkdv_ranges(cu, ops: Operands, G, D, LSE, g, k0, which, noise, scale=None, causal=True,
                per_row_ds=False):
    """Near-midpoint elements of the 32 keys of the block at k0 (kv head g):
    which 0 the P^ of dV, 1 the dS^ of dK; arrays (h, i, j, lo, hi) as in
    dq_ranges."""
    cu = _c(cu, np.int32)
    G, D, LSE = (_c(x, np.float64) for x in (G, D, LSE))
    T, Hq, Hkv, d = ops.T, ops.Hq, ops.Hkv, ops.d
    scale = default_scale(d) if scale is None else scale
    args = [T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale), int(bool(causal)),
            *ops.ptrs(), _p(G), _p(D), _p(LSE), int(bool(per_row_ds)), ctypes.c_double(noise),
            int(g), int(k0), int(which)]
    cap = 4096
    while True:
        oh, oi, oj = (np.zeros(cap, np.int32) for _ in range(3))
        lo, hi = np.zeros(cap), np.zeros(cap)
        n = _load().orc_bwd_dkdv_ranges(*args, ctypes.c_int64(cap), _p(oh), _p(oi), _p(oj),
                                        _p(lo), _p(hi))
        if n < 0:
            raise OracleError("oracle returned %d" % n)
        if n <= cap:
            return oh[:n], oi[:n], oj[:n], lo[:n], hi[:n]
        cap = int(n)


def bwd_prep(cu, dO, O, k_exps, v_exps, Hkv, scale=None, causal=True, block=32):
    """dO quantization, D = dO^ . O and the dQ prescale exponents.
    Returns (do_codes, do_exps, D float64 [Hq][T], kpre int32 [Hq][T])."""
    cu = _c(cu, np.int32)
    dO = _c(dO, np.uint16)
    O = _c(O, np.uint16)
    T, Hq, d = dO.shape
    scale = default_scale(d) if scale is None else scale
    gc = np.empty((T, Hq, d), dtype=np.uint8)
    ge = np.empty((Hq, T), dtype=np.uint8)
    D = np.empty((Hq, T), dtype=np.float64)
    kpre = np.empty((Hq, T), dtype=np.int32)
    _check(_load().orc_bwd_prep(T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale),
                                int(bool(causal)), block, _p(dO), _p(O),
                                _p(_c(k_exps, np.uint8)), _p(_c(v_exps, np.uint8)), _p(gc),
                                _p(ge), _p(D), _p(kpre)))
    return gc, ge, D, kpre


def bwd_prescale_seq(cu, do_exps, k_exps, v_exps, Hkv, d, scale=None):
    """The sequence-wide dQ prescale exponents (test-only negative control):
    int32 [Hq][T] from the sequence-wide maxima of the dO, V and K
    exponents."""
    cu = _c(cu, np.int32)
    do_exps = _c(do_exps, np.uint8)
    Hq, T = do_exps.shape
    scale = default_scale(d) if scale is None else scale
    kpre = np.empty((Hq, T), dtype=np.int32)
    _check(_load().orc_bwd_prescale_seq(T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale),
                                        _p(do_exps), _p(_c(k_exps, np.uint8)),
                                        _p(_c(v_exps, np.uint8)), _p(kpre)))
    return kpre


def doc_blocks(cu, tokens=None):
    """First tokens of the document-local 32-token blocks (all, or those
    holding the given tokens)."""
    cu = np.asarray(cu, dtype=np.int64)
    starts = []
    if tokens is None:
        for b in range(len(cu) - 1):
            starts.extend(range(int(cu[b]), int(cu[b + 1]), 32))
        return np.array(starts, dtype=np.int32)
    for t in tokens:
        b = int(np.searchsorted(cu, t, side="right") - 1)
        while cu[b + 1] <= t:
            b += 1
        starts.append(int(cu[b]) + 32 * ((int(t) - int(cu[b])) // 32))
    return np.array(sorted(set(starts)), dtype=np.int32)


def _pairs(heads, starts):
    heads = np.asarray(heads, dtype=np.int32)
    starts = np.asarray(starts, dtype=np.int32)
    hh, ss = np.meshgrid(heads, starts, indexing="ij")
    return np.ascontiguousarray(np.stack([hh.ravel(), ss.ravel()], axis=1), dtype=np.int32)


def bwd_dq(cu, ops: Operands, G, D, LSE, scale=None, causal=True, mode=MODE_ROUNDED,
           per_row_ds=False, qblocks=None, kpre=None, dq_tile=256):
    """dQ (float64 [T][Hq][d]) for the listed (q head, block start) pairs
    (default: every block of every head).  G: dequantized dO; D: [Hq][T];
    LSE: [Hq][T] natural log as saved by a forward.  With kpre (int32
    [Hq][T] prescale exponents) returns (dQ, dQ16): dQ16 is the same
    gradient through the method's FP16 accumulation (partials per
    document-relative tile of dq_tile keys boosted by 2^(kpre + f), rounded
    to FP16, summed in FP16 in tile order)."""
    cu = _c(cu, np.int32)
    T, Hq, Hkv, d = ops.T, ops.Hq, ops.Hkv, ops.d
    scale = default_scale(d) if scale is None else scale
    if qblocks is None:
        qblocks = _pairs(range(Hq), doc_blocks(cu))
    qblocks = _c(qblocks, np.int32).reshape(-1, 2)
    dQ = np.zeros((T, Hq, d), dtype=np.float64)
    kp = _c(kpre, np.int32) if kpre is not None else None
    dq16 = np.zeros((T, Hq, d), dtype=np.float64) if kpre is not None else None
    _check(_load().orc_bwd_dq(
        T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale), int(bool(causal)),
        *ops.ptrs(), _p(_c(G, np.float64)), _p(_c(D, np.float64)), _p(_c(LSE, np.float64)),
        mode, int(bool(per_row_ds)), ctypes.c_int64(qblocks.shape[0]), _p(qblocks), _p(dQ),
        _p(kp), _p(dq16), int(dq_tile)))
    return (dQ, dq16) if kpre is not None else dQ


def bwd_dkdv(cu, ops: Operands, G, D, LSE, scale=None, causal=True, mode=MODE_ROUNDED,
             per_row_ds=False, kblocks=None):
    """dK, dV (float64 [T][Hkv][d]) for the listed (kv head, block start)
    pairs (default: every block of every kv head)."""
    cu = _c(cu, np.int32)
    T, Hq, Hkv, d = ops.T, ops.Hq, ops.Hkv, ops.d
    scale = default_scale(d) if scale is None else scale
    if kblocks is None:
        kblocks = _pairs(range(Hkv), doc_blocks(cu))
    kblocks = _c(kblocks, np.int32).reshape(-1, 2)
    dK = np.zeros((T, Hkv, d), dtype=np.float64)
    dV = np.zeros((T, Hkv, d), dtype=np.float64)
    _check(_load().orc_bwd_dkdv(
        T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale), int(bool(causal)),
        *ops.ptrs(), _p(_c(G, np.float64)), _p(_c(D, np.float64)), _p(_c(LSE, np.float64)),
        mode, int(bool(per_row_ds)), ctypes.c_int64(kblocks.shape[0]), _p(kblocks), _p(dK),
        _p(dV)))
    return dK, dV


def bwd_block(cu, ops: Operands, G, D, LSE, h, q0, k0, scale=None, causal=True,
              mode=MODE_ROUNDED, per_row_ds=False):
    """One document-local 32x32 block of the recomputed backward.  Returns a
    dict of [32][32] float64 arrays: P, dP, dS, Pq, dSk, dSq."""
    cu = _c(cu, np.int32)
    T, Hq, Hkv, d = ops.T, ops.Hq, ops.Hkv, ops.d
    scale = default_scale(d) if scale is None else scale
    out = {k: np.zeros((32, 32), dtype=np.float64) for k in ("P", "dP", "dS", "Pq", "dSk", "dSq")}
    _check(_load().orc_bwd_block(
        T, len(cu) - 1, _p(cu), Hq, Hkv, d, ctypes.c_double(scale), int(bool(causal)),
        *ops.ptrs(), _p(_c(G, np.float64)), _p(_c(D, np.float64)), _p(_c(LSE, np.float64)),
        mode, int(bool(per_row_ds)), int(h), int(q0), int(k0),
        *[_p(out[k]) for k in ("P", "dP", "dS", "Pq", "dSk", "dSq")]))
    return out
