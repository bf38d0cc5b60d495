"""Start-up cost tables measured on this GPU (vLLM blog "Adaptive Verification in
vLLM", section "The cost model").

At start-up, dummy steps are timed at every captured graph size and at a few sizes
past the largest one; each shape's cost is the median over five timings, and the
costs form two tables (verification indexed by the step's token count, drafting by
the number of requests), each made non-decreasing.  Here the dummy step is a stand-in for the target model's forward
pass -- `layers` bf16 GEMMs of shape [t, H] x [H, H] -- since no model runs in this
package; the timing (dspark_profile_shapes) and the table construction
(dspark_build_cost_table) are the library's.
"""
from __future__ import annotations

import numpy as np

from . import binding as B


def graph_shapes(graph_max: int, above=(1.5, 2.0)) -> list:
    """Powers of two up to graph_max (the captured sizes) plus sizes above it."""
    shapes, g = [], 1
    while g < graph_max:
        shapes.append(g)
        g *= 2
    shapes.append(graph_max)
    shapes += [int(graph_max * f) for f in above if int(graph_max * f) > graph_max]
    return sorted(set(shapes))


class GemmProxy:
    """A token-count-shaped dummy step: `layers` chained [t, H] x [H, H] bf16 GEMMs."""

    def __init__(self, max_tokens: int, hidden: int = 7168, layers: int = 4, device="cuda", seed: int = 0):
        import torch
        g = torch.Generator(device="cpu").manual_seed(seed)
        self.x = (torch.randn((max_tokens, hidden), generator=g) * 0.1).to(device=device, dtype=torch.bfloat16)
        self.w = [(torch.randn((hidden, hidden), generator=g) * (hidden ** -0.5)).to(device=device,
                                                                                    dtype=torch.bfloat16)
                  for _ in range(layers)]
        self.y = [torch.empty_like(self.x) for _ in range(2)]
        self.max_tokens = max_tokens

    def __call__(self, t: int):
        import torch
        if not 1 <= t <= self.max_tokens:
            raise ValueError(f"proxy step of {t} tokens outside [1, {self.max_tokens}]")
        src = self.x[:t]
        for i, w in enumerate(self.w):
            dst = self.y[i % 2][:t]
            torch.matmul(src, w, out=dst)
            src = dst


def measure_table(step, graph_max: int, table_len: int, runs: int = 5, warmup: int = 2, above=(1.5, 2.0)):
    """Profile `step` over graph_shapes(graph_max, above) and build the forced table.
    Returns (table [table_len] float32, shapes, samples [n_shapes, runs])."""
    shapes = graph_shapes(graph_max, above)
    samples = B.dspark_profile_shapes(step, shapes, runs=runs, warmup=warmup)
    table = B.dspark_build_cost_table(shapes, samples, graph_max, table_len)
    return table, shapes, samples
