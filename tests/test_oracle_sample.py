"""Pins of probabilistic draft sampling in the oracle (Gumbel-max over the chained
logits with Philox4x32-10 random numbers).

  * The Philox round structure, at 64-bit words, reproduces numpy's Philox bit
    generator (Philox4x64-10) word for word -- a library routine.
  * The C oracle's Philox4x32-10 and the Python one agree on random counters and keys
    (two implementations written separately).
  * The variates are standard Gumbel (mean = Euler's constant, variance = pi^2 / 6).
  * Sampling frequencies equal softmax(x / temperature) (closed form), at two
    temperatures; a vanishing temperature gives the greedy chain.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import rng as orng
from confidence_scheduled_verification_amd import inputs


def test_philox_structure_matches_numpy_philox4x64():
    r = np.random.default_rng(0)
    for _ in range(20):
        key = [int(x) for x in r.integers(0, 2**63, size=2, dtype=np.uint64)]
        ctr = [int(x) for x in r.integers(0, 2**63, size=4, dtype=np.uint64)]
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
        raw = [int(x) for x in bg.random_raw(4)]
        # numpy advances the 256-bit counter before the first block
        nxt = ctr[:]
        for w in range(4):
            nxt[w] = (nxt[w] + 1) % 2**64
            if nxt[w] != 0:
                break
        assert orng.philox(nxt, key, orng.PHILOX4x64) == raw


def test_c_and_python_philox4x32_agree():
    r = np.random.default_rng(1)
    for _ in range(500):
        ctr = [int(x) for x in r.integers(0, 2**32, size=4, dtype=np.uint64)]
        key = [int(x) for x in r.integers(0, 2**32, size=2, dtype=np.uint64)]
        assert oracle.philox4x32(ctr, key) == orng.philox(ctr, key)
    assert oracle.philox4x32([0, 0, 0, 0], [0, 0]) == orng.philox([0, 0, 0, 0], [0, 0])


def test_variates_are_standard_gumbel():
    g = []
    for c in range(30000):
        for w in orng.philox((c, 7, 3, 0), (12345, 678)):
            g.append(orng.gumbel(w))
    g = np.array(g)
    n = len(g)
    assert abs(g.mean() - 0.5772156649) < 4 * math.sqrt(math.pi ** 2 / 6 / n)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.03
    u = np.array([orng.uniform(w) for w in orng.philox((1, 2, 3, 4), (5, 6))])
    assert np.all((u > 0) & (u < 1)) and np.all(u.astype(np.float32) == u)


@pytest.mark.parametrize("temperature", [1.0, 0.5])
def test_sampling_frequencies_are_softmax(temperature):
    # One position, Bmat = 0 so x = base: every row is the same 6-way choice with its own
    # random numbers (the counter holds the row), so the token counts estimate the law.
    R, V, rank = 60000, 6, 4
    x = np.array([1.0, 0.25, -0.5, 1.5, 0.0, -2.0], np.float32)
    base = np.tile(x, (R, 1)).reshape(R, 1, V)
    A = np.zeros((V, rank), np.float32)
    Bmat = np.zeros((rank, V), np.float32)
    tok, _, _ = oracle.chain_sample(base, A, Bmat, inputs.F32, np.zeros(R, np.int32), temperature, seed=2024)
    counts = np.bincount(tok[:, 0], minlength=V)
    p = np.exp(x.astype(np.float64) / temperature)
    p /= p.sum()
    sd = np.sqrt(R * p * (1 - p))
    assert np.all(np.abs(counts - R * p) < 4.5 * sd), (counts, R * p)


def test_vanishing_temperature_is_the_greedy_chain():
    c = inputs.random_case(3, R=6, K=4, V=300, rank=32, dtype=inputs.BF16)
    greedy, logits, _ = oracle.chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"], want_logits=True)
    # the logits' top-2 gaps dwarf the noise once divided by a tiny temperature
    srt = np.sort(logits, axis=2)
    assert np.all(srt[:, :, -1] - srt[:, :, -2] > 1e-3)
    tok, _, _ = oracle.chain_sample(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"], 1e-6, seed=9)
    np.testing.assert_array_equal(tok, greedy)


def test_sampling_depends_on_seed_and_position_and_keys_the_chain():
    c = inputs.random_case(4, R=8, K=5, V=64, rank=32, dtype=inputs.BF16, base_std=0.5)
    a, pa, _ = oracle.chain_sample(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"], 1.0, seed=1,
                                   want_perturbed=True)
    b, _, _ = oracle.chain_sample(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"], 1.0, seed=2)
    a2, _, _ = oracle.chain_sample(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"], 1.0, seed=1)
    assert np.array_equal(a, a2) and not np.array_equal(a, b)
    assert np.array_equal(a, np.argmax(pa, axis=2))
    # the perturbation at (r, i, v) is the Python generator's variate added to x / temperature
    _, x, _ = oracle.chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"], forced=a, want_logits=True)
    for r, i, v in ((0, 0, 0), (3, 2, 17), (7, 4, 63)):
        assert pa[r, i, v] == x[r, i, v] / 1.0 + orng.gumbel(orng.draft_bits(1, r, i, v))
