"""Seeded synthetic inputs for the attention workloads.

Shared by the tests, the benchmark and the smoke check, for both the HIP path
and the CPU oracle.  This module draws random numbers and packs documents; it
holds none of the method's arithmetic (no quantization, no attention).

Every tensor is drawn with ``numpy.random.default_rng(seed)`` in the fixed
order: document lengths -> Q -> K -> V -> dO -> outlier masks -> per-channel
standard deviations, as float32, then rounded to bfloat16 (nearest, ties to
even) and returned as raw uint16 bit patterns in packed [T][H][d] layout.

The named workloads stand in for the pages' packed causal training shapes
(16 query heads, head dim 128, many documents per packed row) and for their
trained-model activation captures, which are not available here.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FLAG_CAUSAL = 1
FLAG_EXACT = 2
FLAG_FP4_SCORE = 4
FLAG_DETERMINISTIC = 8


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, nearest with ties to even (finite
    inputs only)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1)))
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def doc_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> list[int]:
    """Integer lengths uniform on {lo..hi}, drawn until they reach `total`;
    the last document is cut so the lengths sum to exactly `total`."""
    lens: list[int] = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def cu_from_lengths(lens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


@dataclass
class Workload:
    name: str
    T: int
    cu: np.ndarray
    Hq: int
    Hkv: int
    d: int
    flags: int
    q: np.ndarray = field(repr=False)
    k: np.ndarray = field(repr=False)
    v: np.ndarray = field(repr=False)
    do: np.ndarray = field(repr=False)

    @property
    def causal(self) -> bool:
        return bool(self.flags & FLAG_CAUSAL)

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu.astype(np.int64))

    def visible_pairs(self) -> int:
        n = self.lengths
        return int(np.sum(n * (n + 1) // 2)) if self.causal else int(np.sum(n * n))


def make(name: str, seed: int, T: int, lens, Hq: int, Hkv: int, d: int, flags: int = FLAG_CAUSAL,
         lo_hi=None, do_std: float = 1.0, kv_outlier_frac: float = 0.0,
         kv_outlier_mult: float = 20.0, qk_logstd: tuple | None = None,
         capacity: int | None = None) -> Workload:
    """Generic generator.  Either `lens` (explicit document lengths) or `lo_hi`
    (uniform lengths drawn until T tokens) fixes the packing.  `capacity`
    adds padding rows after the last document (rows beyond cu[B])."""
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = doc_lengths(rng, T, lo_hi[0], lo_hi[1])
    cu = cu_from_lengths(lens)
    assert int(cu[-1]) <= T
    rows = capacity if capacity is not None else T
    q = rng.standard_normal((rows, Hq, d), dtype=np.float32)
    k = rng.standard_normal((rows, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((rows, Hkv, d), dtype=np.float32)
    do = rng.standard_normal((rows, Hq, d), dtype=np.float32)
    if do_std != 1.0:
        do *= np.float32(do_std)
    if kv_outlier_frac > 0.0:
        mk = rng.random((rows, Hkv, d), dtype=np.float32) < kv_outlier_frac
        mv = rng.random((rows, Hkv, d), dtype=np.float32) < kv_outlier_frac
        k[mk] *= np.float32(kv_outlier_mult)
        v[mv] *= np.float32(kv_outlier_mult)
    if qk_logstd is not None:
        lo, hi = np.log(qk_logstd[0]), np.log(qk_logstd[1])
        sq = np.exp(rng.uniform(lo, hi, size=(Hq, d))).astype(np.float32)
        sk = np.exp(rng.uniform(lo, hi, size=(Hkv, d))).astype(np.float32)
        q *= sq[None]
        k *= sk[None]
    return Workload(name, rows, cu, Hq, Hkv, d, flags, f32_to_bf16_bits(q), f32_to_bf16_bits(k),
                    f32_to_bf16_bits(v), f32_to_bf16_bits(do))


# The named workloads.  "tiny" is the small case the oracle finishes in
# seconds; "long_doc" is the headline single-GPU workload; packed MHA, packed
# GQA and the exact option are parity cases timed alongside; the two exact-
# shape rows split the exact option's cost (scale policy, score view); the
# two 65,536-token rows are the packed shapes the pages time a training call
# on, kept as context rows.
def tiny(seed: int = 0) -> Workload:
    """One 256-token document, 1/1 heads, d = 64, causal, N(0, 1)."""
    return make("tiny", seed, 256, [256], 1, 1, 64)


def packed_mha(seed: int = 0) -> Workload:
    """16384 tokens, lengths U{512..4096} (last cut to fit), 16/16 heads,
    d = 128, causal; 1 % of K and V entries x20; dO ~ 1e-2 N(0, 1)."""
    return make("packed_mha", seed, 16384, None, 16, 16, 128, lo_hi=(512, 4096),
                do_std=1e-2, kv_outlier_frac=0.01)


def packed_gqa(seed: int = 0) -> Workload:
    """32768 tokens, lengths U{2048..8192}, 32/8 heads, d = 128, causal,
    dO ~ 1e-2 N(0, 1)."""
    return make("packed_gqa", seed, 32768, None, 32, 8, 128, lo_hi=(2048, 8192), do_std=1e-2)


def long_doc(seed: int = 0) -> Workload:
    """One 65536-token document, 8/8 heads, d = 128, causal; Q and K with a
    per-(head, channel) std log-uniform in [0.1, 10]."""
    return make("long_doc", seed, 65536, [65536], 8, 8, 128, qk_logstd=(0.1, 10.0))


def exact_option(seed: int = 0) -> Workload:
    """8 documents x 2048, 16/4 heads, d = 64; per-token operand scales,
    per-query-row dS exponents and the E2M1 score view."""
    return make("exact_option", seed, 16384, [2048] * 8, 16, 4, 64,
                flags=FLAG_CAUSAL | FLAG_EXACT | FLAG_FP4_SCORE)


def exact_shape_block(seed: int = 0) -> Workload:
    """The exact option's shape and inputs (8 documents x 2048, 16/4 heads,
    d = 64) with token-block operands and FP8 scores: the baseline the
    exact-scale and score-view costs are measured against."""
    return make("exact_shape_block", seed, 16384, [2048] * 8, 16, 4, 64)


def exact_shape_no_fp4(seed: int = 0) -> Workload:
    """The exact option without the E2M1 score view: per-token operand scales
    and per-query-row dS exponents, FP8 scores."""
    return make("exact_shape_no_fp4", seed, 16384, [2048] * 8, 16, 4, 64,
                flags=FLAG_CAUSAL | FLAG_EXACT)


def docs_16x4096(seed: int = 0) -> Workload:
    """16 documents x 4096 tokens (65,536), 16/16 heads, d = 128, causal,
    N(0, 1); dO ~ 1e-2 N(0, 1)."""
    return make("docs_16x4096", seed, 65536, [4096] * 16, 16, 16, 128, do_std=1e-2)


def docs_8192_224x256(seed: int = 0) -> Workload:
    """One 8192-token document then 224 documents of 256 (65,536 tokens),
    16/16 heads, d = 128, causal, N(0, 1); dO ~ 1e-2 N(0, 1)."""
    return make("docs_8192_224x256", seed, 65536, [8192] + [256] * 224, 16, 16, 128, do_std=1e-2)


NAMED = {
    "tiny": tiny,
    "packed_mha": packed_mha,
    "packed_gqa": packed_gqa,
    "long_doc": long_doc,
    "exact_option": exact_option,
    "exact_shape_block": exact_shape_block,
    "exact_shape_no_fp4": exact_shape_no_fp4,
    "docs_16x4096": docs_16x4096,
    "docs_8192_224x256": docs_8192_224x256,
}
