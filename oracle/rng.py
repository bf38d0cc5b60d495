"""ORACLE -- test infrastructure only (tests, smoke check and the CPU-baseline leg).

The counter-based random numbers of probabilistic draft sampling, written from the
published definition of the Philox generators (Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011): an N-word counter is
bijectively scrambled under a 2-word key by R rounds of

    (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0))

with the key bumped by two Weyl constants between rounds.  One implementation for
both word widths: at 64 bits it must reproduce numpy's Philox bit generator (which
is Philox4x64-10), and the draft sampler uses the 32-bit generator Philox4x32-10.

Draft sampling (readings): the drafted token at (r, i)
is a sample from softmax(x / temperature) over the chained logits x (the vLLM blog's
benchmark runs at temperature 1.0, "Results"), drawn by the Gumbel-max rule:
argmax_v x[v] / temperature + g[v] with g[v] = -log(-log u[v]).  u[v] comes from
Philox4x32-10 with counter (v // 4, i, r, 0) and key (seed low word, seed high
word), output word v % 4, of which the top 23 bits b give u = (2 b + 1) / 2^24, a
float32 strictly inside (0, 1).
"""
from __future__ import annotations

import math

PHILOX4x32 = dict(W=32, M=(0xD2511F53, 0xCD9E8D57), K=(0x9E3779B9, 0xBB67AE85))
PHILOX4x64 = dict(W=64, M=(0xD2E7470EE14C6C93, 0xCA5A826395121157), K=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B))


def philox(counter, key, spec=PHILOX4x32, rounds=10):
    """Philox4xW-rounds of a 4-word counter under a 2-word key; returns the 4 output words."""
    W = spec["W"]
    mask = (1 << W) - 1
    M0, M1 = spec["M"]
    K0, K1 = spec["K"]
    c = [int(x) & mask for x in counter]
    k = [int(x) & mask for x in key]
    for _ in range(rounds):
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        c = [(p1 >> W) ^ c[1] ^ k[0], p1 & mask, (p0 >> W) ^ c[3] ^ k[1], p0 & mask]
        k = [(k[0] + K0) & mask, (k[1] + K1) & mask]
    return c


def draft_bits(seed: int, r: int, i: int, v: int) -> int:
    """The 32 random bits of vocabulary entry v at request r, position i."""
    words = philox((v // 4, i, r, 0), (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    return words[v % 4]


def uniform(bits: int) -> float:
    """(2 b + 1) / 2^24 for the top 23 bits b: exactly a float32, strictly inside (0, 1)."""
    return (2 * (bits >> 9) + 1) / float(1 << 24)


def gumbel(bits: int) -> float:
    """A standard Gumbel variate from the bits: -log(-log u)."""
    return -math.log(-math.log(uniform(bits)))
