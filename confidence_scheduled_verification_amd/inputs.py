"""Seeded synthetic workloads for the chain-and-schedule step.

This module is shared by the oracle tests and the HIP path, so it holds only the
input recipe: shapes, seeds, random draws, the bf16 rounding of those draws and
the raw (unforced) synthetic cost profiles.  None of the method's own arithmetic
lives here: survival products, sorting, budget choice, cost-table forcing and the
chained argmax are implemented separately by the oracle and by the HIP library.

Workload shapes follow the pages' deployments:
  * K = 7 draft positions (``num_speculative_tokens`` 7, vLLM blog "Adaptive
    Verification in vLLM", appendix) and K = 15 (DFlash block on the MAX worklog,
    "The boards");
  * rank 256 for the Markov head's factorisation (DSpark summary, "Draft better");
  * first-position confidence around 0.75-0.85 and last-position survival under
    0.1 (vLLM blog, "The problem");
  * concurrency up to 256 (vLLM blog, "Results");
  * a cost staircase from CUDA-graph padding, a 4096 capture limit and a jump past
    it (vLLM blog, "The cost model" and the appendix's capture size).

Random-draw order per workload (numpy ``default_rng(seed)``): base logits, A,
Bmat, prev0, z, eps, cost noise.  Normal draws are float32
``standard_normal`` scaled by the stated standard deviation; bf16 workloads round
those float32 values to nearest-even bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    R: int                 # drafting requests (rows of base / conf)
    R_all: int             # scheduled requests (indexes the draft-cost table)
    n_sampling: int        # requests that sample a bonus token this step
    K: int                 # draft positions per request
    V: int                 # vocabulary
    rank: int              # rank of the Markov-head factorisation
    dtype: int             # F32 or BF16 for base / A / Bmat
    T: int                 # non-draft tokens already scheduled this step
    base_std: float
    factor_std: float
    conf_a: float          # confidence logit offset
    conf_b: float          # confidence logit slope per position
    conf_eps: float        # per-slot noise scale (0 = none)
    verify_len: int        # verify-cost table covers t in [0, verify_len)
    graph_max: int         # largest captured graph size (staircase end)
    verify_base: float     # staircase intercept in microseconds
    verify_slope: float    # microseconds per padded token
    jump_us: float         # extra cost once t passes graph_max
    noise: float           # multiplicative +-noise on the verify table
    seed: int
    has_chain: bool = True

    @property
    def draft_len(self) -> int:
        return max(self.R_all, 256) + 1

    @property
    def n_slots(self) -> int:
        return self.R * self.K


WORKLOADS = {
    "tiny": Workload("tiny", R=4, R_all=4, n_sampling=4, K=7, V=1024, rank=16, dtype=F32, T=0,
                     base_std=1.0, factor_std=0.1, conf_a=1.5, conf_b=0.45, conf_eps=0.0,
                     verify_len=65, graph_max=64, verify_base=2000.0, verify_slope=1.5,
                     jump_us=0.0, noise=0.0, seed=0),
    "small": Workload("small", R=32, R_all=32, n_sampling=32, K=7, V=32768, rank=256, dtype=BF16, T=0,
                      base_std=2.0, factor_std=0.05, conf_a=1.5, conf_b=0.45, conf_eps=0.3,
                      verify_len=513, graph_max=512, verify_base=2000.0, verify_slope=1.2,
                      jump_us=0.0, noise=0.0, seed=1),
    "mid": Workload("mid", R=112, R_all=128, n_sampling=112, K=7, V=129280, rank=256, dtype=BF16, T=2048,
                    base_std=2.0, factor_std=0.05, conf_a=1.5, conf_b=0.45, conf_eps=0.3,
                    verify_len=8193, graph_max=4096, verify_base=2000.0, verify_slope=1.0,
                    jump_us=3000.0, noise=0.03, seed=2),
    "headline": Workload("headline", R=256, R_all=256, n_sampling=256, K=7, V=129280, rank=256, dtype=BF16,
                         T=0, base_std=2.0, factor_std=0.05, conf_a=1.5, conf_b=0.45, conf_eps=0.3,
                         verify_len=8193, graph_max=4096, verify_base=2000.0, verify_slope=1.0,
                         jump_us=3000.0, noise=0.03, seed=3),
    "large": Workload("large", R=64, R_all=64, n_sampling=64, K=15, V=262144, rank=256, dtype=BF16, T=512,
                      base_std=2.0, factor_std=0.05, conf_a=2.0, conf_b=0.35, conf_eps=0.3,
                      verify_len=16385, graph_max=4096, verify_base=2000.0, verify_slope=1.0,
                      jump_us=3000.0, noise=0.0, seed=4),
    # one GPU's share of the headline chain under an 8-way vocabulary split (tensor
    # parallelism 8, as the vLLM blog's "Results" deployment): V / 8 columns, every request
    "shard": Workload("shard", R=256, R_all=256, n_sampling=256, K=7, V=16160, rank=256, dtype=BF16,
                      T=0, base_std=2.0, factor_std=0.05, conf_a=1.5, conf_b=0.45, conf_eps=0.3,
                      verify_len=8193, graph_max=4096, verify_base=2000.0, verify_slope=1.0,
                      jump_us=3000.0, noise=0.03, seed=5),
    # scheduler-only sweep: 1024 requests x 15 positions, same confidence law and tables as "large"
    "sweep": Workload("sweep", R=1024, R_all=1024, n_sampling=1024, K=15, V=0, rank=0, dtype=BF16, T=512,
                      base_std=0.0, factor_std=0.0, conf_a=2.0, conf_b=0.35, conf_eps=0.3,
                      verify_len=16385, graph_max=4096, verify_base=2000.0, verify_slope=1.0,
                      jump_us=3000.0, noise=0.0, seed=4, has_chain=False),
}


def pad_to_graph(t: int, graph_max: int) -> int:
    """Smallest captured graph size (a power of two) that holds t tokens.

    121 tokens are padded up to the 128-token graph (vLLM blog, "The cost model").
    pad(0) is the smallest graph, 1.  Sizes above graph_max are not padded.
    """
    if t > graph_max:
        return t
    g = 1
    while g < t:
        g *= 2
    return g


def raw_verify_cost(w: Workload, rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """Synthetic profiled verification cost (microseconds) for t in [0, verify_len), before forcing.

    Inside the capture region the cost is a staircase over padded sizes; past it the cost
    is continuous and carries a jump (vLLM blog, "The cost model").  Optional multiplicative
    noise stands in for profiling noise.
    """
    t = np.arange(w.verify_len)
    padded = np.array([pad_to_graph(int(x), w.graph_max) for x in t], dtype=np.float64)
    cost = w.verify_base + w.verify_slope * padded
    cost = np.where(t > w.graph_max, cost + w.jump_us, cost)
    if w.noise > 0.0:
        assert rng is not None
        cost = cost * (1.0 + rng.uniform(-w.noise, w.noise, size=w.verify_len))
    return cost.astype(np.float32)


def raw_draft_cost(w: Workload) -> np.ndarray:
    """Synthetic drafter cost (microseconds) indexed by request count: 300 + 2 n."""
    n = np.arange(w.draft_len, dtype=np.float64)
    return (300.0 + 2.0 * n).astype(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _store(w: Workload, x: np.ndarray) -> np.ndarray:
    return round_to_bf16(x) if w.dtype == BF16 else x.astype(np.float32)


def _confidences(w: Workload, rng: np.random.Generator) -> np.ndarray:
    z = rng.standard_normal(w.R)
    i = np.arange(w.K)
    logit = z[:, None] + w.conf_a - w.conf_b * i[None, :]
    if w.conf_eps > 0.0:
        logit = logit + w.conf_eps * rng.standard_normal((w.R, w.K))
    return (1.0 / (1.0 + np.exp(-logit))).astype(np.float32)


@dataclasses.dataclass
class Inputs:
    """One step's host inputs.  base/A/Bmat are uint16 bf16 bit patterns or float32."""
    w: Workload
    base: Optional[np.ndarray]      # [R, K, V]
    A: Optional[np.ndarray]         # [V, rank]
    Bmat: Optional[np.ndarray]      # [rank, V]
    prev0: Optional[np.ndarray]     # [R] int32
    conf: np.ndarray                # [R, K] float32
    verify_cost_raw: np.ndarray     # [verify_len] float32, unforced
    draft_cost_raw: np.ndarray      # [draft_len] float32, unforced


def generate(w: Workload) -> Inputs:
    """The workload's fixed inputs (seed = workload seed)."""
    rng = np.random.default_rng(w.seed)
    base = A = Bmat = prev0 = None
    if w.has_chain:
        base = _store(w, _normal(rng, (w.R, w.K, w.V), w.base_std))
        A = _store(w, _normal(rng, (w.V, w.rank), w.factor_std))
        Bmat = _store(w, _normal(rng, (w.rank, w.V), w.factor_std))
        prev0 = rng.integers(0, w.V, size=w.R, dtype=np.int32)
    conf = _confidences(w, rng)
    vc = raw_verify_cost(w, rng)
    dc = raw_draft_cost(w)
    return Inputs(w, base, A, Bmat, prev0, conf, vc, dc)


def step_seed(w: Workload, k: int) -> int:
    """Seed of step k in a multi-step run: weights and tables stay, per-step inputs are redrawn."""
    return w.seed * 1_000_003 + k


def generate_step(w: Workload, k: int) -> dict:
    """Per-step inputs of step k (base logits, prev0, confidences) for multi-step runs."""
    rng = np.random.default_rng(step_seed(w, k))
    out = {}
    if w.has_chain:
        out["base"] = _store(w, _normal(rng, (w.R, w.K, w.V), w.base_std))
        out["prev0"] = rng.integers(0, w.V, size=w.R, dtype=np.int32)
    out["conf"] = _confidences(w, rng)
    return out


def random_case(seed: int, R: int, K: int, V: int, rank: int, dtype: int, base_std=2.0, factor_std=0.05,
                conf_a=1.5, conf_b=0.45, conf_eps=0.3) -> dict:
    """Small ad-hoc case (ragged shapes for parity tests): base, A, Bmat, prev0, conf."""
    rng = np.random.default_rng(seed)
    w = dataclasses.replace(WORKLOADS["small"], R=R, K=K, V=V, rank=rank, dtype=dtype,
                            conf_a=conf_a, conf_b=conf_b, conf_eps=conf_eps)
    base = _store(w, _normal(rng, (R, K, V), base_std))
    A = _store(w, _normal(rng, (V, rank), factor_std))
    Bmat = _store(w, _normal(rng, (rank, V), factor_std))
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    conf = _confidences(w, rng)
    return dict(base=base, A=A, Bmat=Bmat, prev0=prev0, conf=conf)


def synthetic_target(ver_tokens, offsets, conf, V: int, seed: int) -> np.ndarray:
    """Stand-in for the target model's greedy tokens over one step's verified drafts.

    For request r with verified drafts d_0..d_{L-1} (ver_tokens[offsets[r]:offsets[r+1]])
    the target's token at entry j < L equals d_j with probability conf[r, j] and is some
    other token otherwise; entry L is a uniform token.  Entries sit at offsets[r] + r + j
    (1 + L per request) in a buffer of R*K + R tokens (unused entries 0).  Acceptance is
    thereby drawn from the confidences: the chance that drafts 0..i all match is the
    product of conf[r, 0..i].  All draws are made up front, so the stream does not depend
    on the allocation."""
    ver_tokens = np.asarray(ver_tokens).reshape(-1)
    offsets = np.asarray(offsets).reshape(-1)
    conf = np.asarray(conf, dtype=np.float64)
    R, K = conf.shape
    rng = np.random.default_rng(seed)
    u = rng.random((R, K))
    other = rng.integers(1, max(V, 2), size=(R, K))
    bonus = rng.integers(0, V, size=R)
    target = np.zeros(R * K + R, dtype=np.int32)
    for r in range(R):
        o, L = int(offsets[r]), int(offsets[r + 1] - offsets[r])
        for j in range(L):
            d = int(ver_tokens[o + j])
            target[o + r + j] = d if u[r, j] < conf[r, j] else (d + int(other[r, j])) % V
        target[o + r + L] = bonus[r]
    return target
