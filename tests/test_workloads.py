"""Seeded inputs and the counting formulas the benchmark uses (no GPU)."""
from __future__ import annotations

import json
import os

import numpy as np

import workloads
from workloads import WORKLOADS, Workload, draw

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_counts.json")


def test_draws_are_deterministic():
    a1, b1, c1 = draw(33, 17, 9, "uniform", 3, True)
    a2, b2, c2 = draw(33, 17, 9, "uniform", 3, True)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2) and np.array_equal(c1, c2)
    a3, _, _ = draw(33, 17, 9, "uniform", 4, True)
    assert not np.array_equal(a1, a3)


def test_draw_order_a_then_b_then_c():
    """B depends only on the seed and A's size: drawing C does not change A or B."""
    a1, b1, _ = draw(20, 10, 30, "uniform", 5, False)
    a2, b2, c2 = draw(20, 10, 30, "uniform", 5, True)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2) and c2 is not None


def test_distributions():
    A, B, C = draw(300, 200, 400, "uniform", 0, True)
    for x in (A, B, C):
        assert x.dtype == np.float32 and x.flags.c_contiguous
        assert x.min() >= -1 and x.max() <= 1 and abs(float(x.mean())) < 0.02
    A, B, C = draw(300, 200, 400, "int4", 2, True)
    for x in (A, B, C):
        assert set(np.unique(x)) == set(np.arange(-4, 5, dtype=np.float32))
    A, B, _ = draw(512, 512, 4096, "mlp", 4, False)
    assert abs(float(A.std()) - 1) < 0.01
    assert abs(float(B.std()) * 64 - 1) < 0.01
    A, B, _ = draw(64, 64, 256, "probe", 5, False)
    assert np.all(np.rint(A.astype(np.float64) * 2 ** 16) == A.astype(np.float64) * 2 ** 16)
    assert set(np.unique(B)) == {-1.0, 0.0, 1.0}


def test_padded_view():
    x = np.arange(12, dtype=np.float32).reshape(3, 4)
    v = workloads.padded(x, 3, np.nan)
    assert np.array_equal(v, x) and v.strides[0] == 7 * 4
    assert np.isnan(v.base[:, 4:]).all()


def test_named_shapes():
    w = WORKLOADS["mlp_up"]
    assert (w.M, w.K, w.N) == (8192, 4096, 14336)
    w = WORKLOADS["mlp_down"]
    assert (w.M, w.K, w.N) == (8192, 14336, 4096)
    w = WORKLOADS["mlp_decode16"]
    assert (w.M, w.K, w.N) == (16, 4096, 14336)
    assert [WORKLOADS[f"sweep{n}"].M for n in (128, 256, 512, 1024, 2048, 4096, 8192)] == \
        [128, 256, 512, 1024, 2048, 4096, 8192]


def test_counts_match_the_pages():
    g = json.load(open(GOLDEN))
    w = WORKLOADS["square4096"]
    assert round(w.flops / 1e9) == g["flops_4096_billion"]["value"]
    # the pages truncate 16.78 million to 16.7
    assert int(w.M * w.N / 1e5) / 10 == g["cells_4096_million"]["value"]
    abc = 4 * (w.M * w.K + w.K * w.N + w.M * w.N)   # A + B + C, as the page counts it
    assert round(abc / 1e6) == g["abc_megabytes_4096"]["value"]
    ai = w.flops / abc
    assert abs(ai / g["arithmetic_intensity_4096"]["value"] - 1) < g["arithmetic_intensity_4096"]["rel_tol"]
    assert 2 * w.K == g["naive_flops_per_thread"]["value"]
    assert 2 * w.K * 4 / 1024 == g["naive_kilobytes_per_thread"]["value"]
    total = w.M * w.N * 2 * w.K * 4 / 1e12
    assert abs(total / g["naive_total_terabytes"]["value"] - 1) < g["naive_total_terabytes"]["rel_tol"]
    # algorithmic bytes of the benchmark (C written once, not read: beta = 0)
    assert w.min_bytes == abc


def test_ladder_times_are_two_mnk_over_rate():
    """Every printed ms equals 2*4096^3 / GFLOP/s: FLOP = 2MNK, epilogue uncounted."""
    g = json.load(open(GOLDEN))
    flops = WORKLOADS["square4096"].flops
    for row in g["ladder"]["rows"]:
        ms = flops / (row["gflops"] * 1e9) * 1e3
        assert abs(ms - row["ms"]) <= 0.051 + 0.001 * row["ms"], row


def test_sector_counts():
    """32 lanes reading 4-byte floats: a warp whose addresses are 16 KB apart
    touches 32 sectors of 32 B (plus 1 for the broadcast operand); one whose
    addresses are consecutive touches 128/32 = 4 (plus 1)."""
    g = json.load(open(GOLDEN))["sectors_per_tick"]
    lanes, fbytes, sector = 32, 4, 32
    strided = len({(lane * 4096 * fbytes) // sector for lane in range(lanes)})
    packed = len({(lane * fbytes) // sector for lane in range(lanes)})
    assert strided + 1 == g["naive"] and packed + 1 == g["swapped"]


def test_min_bytes_counts_c_read_only_with_beta():
    assert Workload("x", 2, 3, 4, 1.0, 0.0, "uniform", 0).min_bytes == 4 * (8 + 12 + 6)
    assert Workload("x", 2, 3, 4, 1.0, 1.0, "uniform", 0).min_bytes == 4 * (8 + 12 + 12)
