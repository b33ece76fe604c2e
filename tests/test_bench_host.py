"""Host checks of the benchmark's algorithmic work counts, the numerators of
every TFLOP/s and GB/s figure it reports, against counts derived here from
the shapes alone: a Newton-Schulz iteration on an m x n matrix (m <= n) is
A = X X^T (symmetric: m(m+1)/2 dot products of length n), B = b A + c A A
(symmetric: m(m+1)/2 dot products of length m) and B X (m n dot products of
length m), two flops per multiply-add; three dense GEMMs would be 2 m^2 n,
2 m^3 and 2 m^2 n.  No GPU."""
import importlib.util
import os

import pytest

from optimizer_muon_step_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _brute_counts(shapes):
    """Dot products counted one by one (tiny shapes only)."""
    gram = poly = upd = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        for i in range(m):
            for j in range(i, m):  # upper triangle, diagonal included
                gram += 2 * n
                poly += 2 * m
        upd += m * n * 2 * m
    return gram, poly, upd


def test_flop_counts_match_dot_product_counts(bench):
    shapes = [(3, 5), (5, 3), (1, 1), (4, 4), (2, 9)]
    assert bench.ns_flops(shapes) == _brute_counts(shapes)
    dense = sum(2 * min(s) ** 2 * max(s) * 2 + 2 * min(s) ** 3 for s in shapes)
    assert bench.ns_flops_dense(shapes) == dense


@pytest.mark.parametrize("config,sym_tflop,dense_tflop", [
    ("c1", 0.00059, 0.00084),
    ("c2", 0.0906, 0.1268),
    ("c3", 1.0877, 1.5220),
    ("c4", 39.33, 55.05),
    ("c5", 0.456, 0.611),
])
def test_per_step_totals_of_the_named_workloads(bench, config, sym_tflop, dense_tflop):
    """Five iterations per step; the totals as the scope table of the
    workloads states them (to its printed precision)."""
    shapes = [(s.rows, s.cols) for s in wl.config_specs(config)]
    sym = 5 * sum(bench.ns_flops(shapes)) / 1e12
    dense = 5 * bench.ns_flops_dense(shapes) / 1e12
    assert sym == pytest.approx(sym_tflop, rel=6e-3)
    assert dense == pytest.approx(dense_tflop, rel=6e-3)


def test_elementwise_bytes_of_the_headline_set():
    """Momentum 12, cast 10 and apply 10 bytes per parameter: 2.72 GB per
    step on the 84.9 M parameters of the GPT-2-124M hidden set."""
    n = sum(s.rows * s.cols for s in wl.config_specs("c3"))
    assert n == 84_934_656
    assert round((12 + 10 + 10) * n / 1e9, 2) == 2.72
