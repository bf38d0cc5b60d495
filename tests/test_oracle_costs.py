"""Pins of the cost-table builder oracle, and the library's host-side builder against it.

Pinned by library routines (np.median), the pages' worked padding example
(tests/golden/pad_graph.json), closed forms (exact lines past the capture limit), and
by rebuilding the synthetic workloads' own cost curves from samples taken at the
profiled shapes."""
import json
import os

import numpy as np
import pytest

from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import costmodel, inputs
from oracle import costs, sched

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_median_is_numpy_median():
    rng = np.random.default_rng(1)
    for n in (1, 2, 5, 6, 9):
        x = rng.normal(100.0, 5.0, size=n).astype(np.float32)
        assert costs.median(x) == float(np.median(x.astype(np.float64))), n


def test_staircase_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "pad_graph.json")))
    shapes = costmodel.graph_shapes(g["graph_max"])
    assert shapes[-2:] == [6144, 8192]
    samples = np.array([[1000.0 + s] * 5 for s in shapes], dtype=np.float32)
    table = costs.build_cost_table(shapes, samples, g["graph_max"], 200)
    assert table[g["tokens"]] == 1000.0 + g["graph"]
    assert table[0] == table[1] == 1001.0 and table[64] == 1064.0 and table[65] == 1128.0


def test_line_past_the_capture_limit_is_exact():
    # eager costs on a line a + b t are reproduced exactly at every t above graph_max, also
    # below the first and beyond the last measured shape
    shapes = [1, 2, 4, 8, 16, 24, 40]
    a, b = 700.0, 3.0
    samples = np.array([[5.0 * s] * 3 if s <= 16 else [a + b * s] * 3 for s in shapes], dtype=np.float32)
    table = costs.build_cost_table(shapes, samples, 16, 60)
    t = np.arange(17, 60)
    np.testing.assert_array_equal(table[17:], (a + b * t).astype(np.float32))
    one = costs.build_cost_table(shapes[:6], samples[:6], 16, 30)     # a single eager shape: constant
    assert np.all(one[17:] == np.float32(a + b * 24))


@pytest.mark.parametrize("name", ["tiny", "small", "mid", "headline", "large"])
def test_rebuilding_the_workload_curves(name):
    # Sampling the workload's noise-free curve at the profiled shapes and rebuilding gives the
    # forced curve back exactly: a staircase over the captured sizes and a line with a jump past it.
    import dataclasses
    w = dataclasses.replace(inputs.WORKLOADS[name], noise=0.0)
    curve = inputs.raw_verify_cost(w)
    shapes = [s for s in costmodel.graph_shapes(w.graph_max, above=(1.25, 1.5, 2.0)) if s < w.verify_len]
    samples = np.repeat(curve[shapes][:, None], 5, axis=1)
    rebuilt = costs.build_cost_table(shapes, samples, w.graph_max, w.verify_len)
    np.testing.assert_array_equal(rebuilt, sched.force_monotone(curve))


def test_median_of_noisy_runs_and_forcing():
    rng = np.random.default_rng(3)
    shapes = costmodel.graph_shapes(64)
    true = np.array([500.0 + 2.0 * s for s in shapes])
    samples = (true[:, None] * (1.0 + rng.uniform(-0.05, 0.05, size=(len(shapes), 5)))).astype(np.float32)
    samples[2, 0] = 1e6                                   # one outlier run: the median ignores it
    table = costs.build_cost_table(shapes, samples, 64, 129)
    assert np.all(np.diff(table) >= 0)
    assert table[4] < 600.0
    assert table[4] == np.float32(np.median(samples[2].astype(np.float64)))


def test_bad_inputs_are_rejected():
    s = np.ones((3, 5), np.float32)
    with pytest.raises(ValueError):
        costs.build_cost_table([1, 2, 2], s, 2, 3)         # not increasing
    with pytest.raises(ValueError):
        costs.build_cost_table([1, 2, 3], s, 4, 4)         # graph_max not measured
    with pytest.raises(ValueError):
        costs.build_cost_table([1, 2, 4], s, 4, 9)         # nothing above graph_max
    bad = s.copy()
    bad[1, 2] = np.nan                                    # any non-finite run, even one the median would skip
    with pytest.raises(ValueError):
        costs.build_cost_table([1, 2, 4], bad, 4, 5)


# ---------------------------------------------------------------- the library's builder (host code)

@pytest.mark.parametrize("runs", [5, 4, 1])
def test_library_builder_matches_the_oracle(runs):
    rng = np.random.default_rng(runs)
    for graph_max, tlen, above in ((64, 129, (1.5, 2.0)), (4096, 8193, (1.5, 2.0)), (512, 513, ()),
                                   (16, 100, (1.25, 3.0, 5.0)), (1, 7, (2.0, 4.0))):
        shapes = costmodel.graph_shapes(graph_max, above)
        base = np.array([2000.0 + 1.3 * s + (900.0 if s > graph_max else 0.0) for s in shapes])
        samples = (base[:, None] * (1.0 + rng.uniform(-0.03, 0.03, size=(len(shapes), runs)))).astype(np.float32)
        want = costs.build_cost_table(shapes, samples, graph_max, tlen)
        got = B.dspark_build_cost_table(shapes, samples, graph_max, tlen)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_library_builder_rejects_what_the_oracle_rejects():
    s = np.ones((3, 5), np.float32)
    for shapes, gm, tlen in (([1, 2, 2], 2, 3), ([1, 2, 3], 4, 4), ([1, 2, 4], 4, 9)):
        with pytest.raises(B.DSparkError):
            B.dspark_build_cost_table(shapes, s, gm, tlen)
    bad = s.copy()
    bad[1, 4] = np.inf
    with pytest.raises(B.DSparkError, match="non-finite"):
        B.dspark_build_cost_table([1, 2, 4], bad, 4, 5)
