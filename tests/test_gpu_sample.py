"""GPU parity of probabilistic draft sampling (dspark_chain_sample): Gumbel-max over the
chained logits with Philox4x32-10 random numbers, against the oracle's sampled chain
under the same seed (teacher forced; a token may differ only where the oracle's two
perturbed values are within the logit tolerance), plus the sampling law itself."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import inputs

pytestmark = pytest.mark.gpu


def _sample(ch, temperature, seed, want_logits=False):
    tokens = torch.full((ch.R, ch.K), -7, dtype=torch.int32, device=gu.DEV)
    logits = torch.empty((ch.R, ch.K, ch.V), dtype=torch.float32, device=gu.DEV) if want_logits else None
    status = torch.zeros(1, dtype=torch.int32, device=gu.DEV)
    B.dspark_chain_sample(ch.base, ch.markov, ch.prev0, temperature, seed, tokens, logits, status, ch.ws)
    torch.cuda.synchronize()
    return tokens.cpu().numpy(), (None if logits is None else logits.cpu().numpy()), int(status.item())


CASES = [  # (R, K, V, rank, dtype, temperature)
    (4, 7, 1024, 32, inputs.BF16, 1.0),
    (37, 5, 1000, 64, inputs.BF16, 1.0),      # ragged V, partial request block
    (300, 3, 2048, 256, inputs.BF16, 0.7),    # more than one request chunk
    (16, 6, 777, 32, inputs.BF16, 2.5),
    (5, 4, 513, 16, inputs.F32, 1.0),
]


@pytest.mark.parametrize("R,K,V,rank,dtype,temperature", CASES)
def test_sampled_chain_matches_the_oracle(R, K, V, rank, dtype, temperature):
    gu.say(f"sample R={R} K={K} V={V} rank={rank} dtype={dtype} T={temperature}")
    c = inputs.random_case(R * 31 + V, R=R, K=K, V=V, rank=rank, dtype=dtype, base_std=1.0)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], dtype, c["prev0"])
    seed = 0x123456789ABCDEF0 + R
    tok, lg, st = _sample(ch, temperature, seed, want_logits=True)
    assert st == 0
    near = gu.assert_chain_parity(tok, lg, c["base"], c["A"], c["Bmat"], dtype, c["prev0"],
                                  sample=(temperature, seed))
    assert near <= max(1, R * K // 50)
    # same seed, same tokens; another seed, other tokens; the greedy chain differs too
    again, _, _ = _sample(ch, temperature, seed)
    np.testing.assert_array_equal(again, tok)
    other, _, _ = _sample(ch, temperature, seed + 1)
    assert not np.array_equal(other, tok)
    greedy, _, _ = ch.run()
    assert not np.array_equal(greedy.cpu().numpy(), tok)


def test_headline_shape_sampled_rows():
    w = inputs.WORKLOADS["headline"]
    ins = inputs.generate(w)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    tok, _, st = _sample(ch, 1.0, 77)
    assert st == 0
    gu.say(f"headline sampled: oracle on all {w.R} rows")
    near = gu.assert_chain_parity(tok, None, ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0, sample=(1.0, 77))
    gu.say(f"headline sampled: every row ok ({near} near-ties)")


@pytest.mark.parametrize("temperature", [1.0, 0.5])
def test_sampling_frequencies_are_softmax(temperature):
    # one position, Bmat = 0 so x = base; every row draws its own numbers from the counter
    R, V, rank = 20000, 6, 32
    x = np.array([1.0, 0.25, -0.5, 1.5, 0.0, -2.0], np.float32)
    base = inputs.round_to_bf16(np.tile(x, (R, 1)).reshape(R, 1, V))
    A = inputs.round_to_bf16(np.zeros((V, rank), np.float32))
    Bmat = inputs.round_to_bf16(np.zeros((rank, V), np.float32))
    ch = gu.Chain(base, A, Bmat, inputs.BF16, np.zeros(R, np.int32))
    tok, _, _ = _sample(ch, temperature, 2024)
    counts = np.bincount(tok[:, 0], minlength=V)
    p = np.exp(inputs.bf16_to_f32(base[0, 0]).astype(np.float64) / temperature)
    p /= p.sum()
    sd = np.sqrt(R * p * (1 - p))
    assert np.all(np.abs(counts - R * p) < 4.5 * sd), (counts, R * p)
