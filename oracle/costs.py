"""ORACLE -- test infrastructure only (tests, smoke check and the CPU-baseline leg).

The start-up cost-table builder, written out plainly (vLLM blog "Adaptive
Verification in vLLM", section "The cost model"): dummy steps are timed over a
fixed set of shapes -- the captured graph sizes plus a couple of sizes above the
largest -- five runs each; the median of each shape's runs is its cost; inside
the capture range a step of t tokens runs (and pays for) the smallest captured
graph that holds it, so the table is a staircase; past the capture limit the cost
is continuous; and the finished table is forced monotone.

Readings:
  * the median of an even number of runs is the mean of the two middle ones
    (computed in double);
  * shapes <= graph_max are the captured graph sizes and must include graph_max;
    entry t <= graph_max takes the median of the smallest captured shape >= t,
    with t = 0 read as 1 (the smallest graph);
  * entry t > graph_max is the straight line through the two nearest measured
    shapes above graph_max: between two of them it interpolates, below the first
    and above the last it extends the first or last segment, and a single such
    shape gives a constant.  In double, in this order:
    c_a + ((c_b - c_a) * (t - s_a)) / (s_b - s_a), then rounded to float32;
  * every entry is then rounded to float32 and the table forced monotone (each
    entry the running maximum of the entries up to it).
"""
from __future__ import annotations

import numpy as np

from oracle import sched


def median(values):
    """The middle value of the sorted runs; for an even count the mean of the two middle ones."""
    v = sorted(float(np.float32(x)) for x in values)
    n = len(v)
    if n == 0:
        raise ValueError("no runs")
    if n % 2 == 1:
        return v[n // 2]
    return (v[n // 2 - 1] + v[n // 2]) / 2.0


def build_cost_table(shapes, samples, graph_max, table_len):
    """shapes [n] strictly increasing positive token (or request) counts, samples [n, runs]
    microseconds.  Returns the forced float32 table of table_len entries."""
    shapes = [int(s) for s in shapes]
    samples = np.asarray(samples, dtype=np.float32)
    if len(shapes) == 0 or samples.shape[0] != len(shapes) or any(s <= 0 for s in shapes):
        raise ValueError("shapes must be positive and match the samples")
    if any(shapes[i] >= shapes[i + 1] for i in range(len(shapes) - 1)):
        raise ValueError("shapes must be strictly increasing")
    if not np.all(np.isfinite(samples)):
        raise ValueError("non-finite sample")
    med = [median(samples[i]) for i in range(len(shapes))]
    captured = [i for i, s in enumerate(shapes) if s <= graph_max]
    eager = [i for i, s in enumerate(shapes) if s > graph_max]
    if not captured or shapes[captured[-1]] != graph_max:
        raise ValueError("the captured shapes must include graph_max")
    if table_len - 1 > graph_max and not eager:
        raise ValueError("entries above graph_max need a measured shape above it")
    raw = []
    for t in range(table_len):
        if t <= graph_max:
            want = max(t, 1)
            g = min(i for i in captured if shapes[i] >= want)
            raw.append(med[g])
        elif len(eager) == 1:
            raw.append(med[eager[0]])
        else:
            # the segment: the two consecutive measured shapes around t, or the end segment
            a = eager[0]
            for i in eager[:-1]:
                if shapes[i] <= t:
                    a = i
            b = eager[eager.index(a) + 1]
            sa, sb, ca, cb = shapes[a], shapes[b], med[a], med[b]
            raw.append(ca + ((cb - ca) * (t - sa)) / (sb - sa))
    return sched.force_monotone(np.array(raw, dtype=np.float64).astype(np.float32))
