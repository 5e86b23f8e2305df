"""Pins of the visible-pair FLOP convention, the generators and the
comparison metrics (CPU only)."""
import numpy as np

import workloads
from oracle import metrics


def test_visible_pair_counts(golden):
    for case in golden("visible_pairs.json")["cases"]:
        lens = []
        for n, count in case["lengths"].items():
            lens += [int(n)] * count
        assert sum(lens) == case["tokens"]
        w = workloads.Workload("x", sum(lens), workloads.cu_from_lengths(lens), 1, 1, 8,
                               workloads.FLAG_CAUSAL, None, None, None, None)
        assert w.visible_pairs() == case["visible_pairs"]


def test_small_gradient_metric(golden):
    g = golden("small_gradient_metric.json")
    ref = np.array([g["big"]] + [g["small"]] * g["n_small"])
    got = ref.copy()
    got[1:] = 0.0
    assert abs(metrics.rel_l2(got, ref) - g["rel_l2_about"]) < 1e-3
    assert abs(metrics.cosine(got, ref) - g["cosine_about"]) < 1e-5
    assert metrics.zero_fraction(got, ref) == g["n_small"] / (g["n_small"] + 1)


def test_doc_length_rule_and_determinism():
    rng = np.random.default_rng(0)
    lens = workloads.doc_lengths(rng, 16384, 512, 4096)
    assert sum(lens) == 16384 and all(n <= 4096 for n in lens)
    assert all(512 <= n for n in lens[:-1])
    a = workloads.make("a", 3, 300, None, 2, 1, 16, lo_hi=(10, 90))
    b = workloads.make("a", 3, 300, None, 2, 1, 16, lo_hi=(10, 90))
    assert np.array_equal(a.cu, b.cu) and np.array_equal(a.q, b.q) and np.array_equal(a.do, b.do)


def test_row_relative_error_floor():
    ref = np.array([[1.0, 2.0], [0.0, 0.0], [1e-9, 0.0]])
    got = ref + np.array([[0.1, 0.0], [1e-4, 0.0], [0.0, 0.0]])
    rr = metrics.row_rel_err(got, ref)
    assert np.allclose(rr, [0.05, 1e-4 / 2e-3, 0.0])
