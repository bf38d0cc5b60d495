"""GPU parity of stage 1 (chain) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["pruned", "dense"])
def form(request):
    """Every chain test runs in both forms of stage 1 (the fp32 tests take the same fp32
    kernels in both)."""
    with gu.chain_form(gu.FORMS[request.param]):
        yield request.param


def _case(seed, R, K, V, rank, dtype, **kw):
    return inputs.random_case(seed, R=R, K=K, V=V, rank=rank, dtype=dtype, **kw)


def test_tiny_workload_fp32_full_parity():
    w = inputs.WORKLOADS["tiny"]
    ins = inputs.generate(w)
    gu.say(f"tiny fp32 R={w.R} K={w.K} V={w.V} rank={w.rank}")
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    tok, lg, st = ch.run(want_logits=True)
    assert st == 0
    near = gu.assert_chain_parity(tok.cpu().numpy(), lg.cpu().numpy(), ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    assert near == 0


def test_small_workload_bf16_full_parity():
    w = inputs.WORKLOADS["small"]
    ins = inputs.generate(w)
    gu.say(f"small bf16 R={w.R} K={w.K} V={w.V} rank={w.rank}")
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    tok, lg, st = ch.run(want_logits=True)
    assert st == 0
    near = gu.assert_chain_parity(tok.cpu().numpy(), lg.cpu().numpy(), ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    assert near <= 1


@pytest.mark.parametrize("R,K,V,rank", [
    (5, 3, 1000, 64),      # V not a multiple of 8 (element-wise loads), partial request block
    (17, 2, 4104, 32),     # two request blocks, ragged vocabulary tile, rank 32
    (33, 4, 777, 96),      # rank 96 padded to 128, short vocabulary
    (300, 2, 2048, 256),   # more requests than one LDS chunk (256)
    (1, 1, 1, 32),         # one vocabulary entry
    (16, 7, 1280 * 8, 128),
])
def test_ragged_bf16_parity(R, K, V, rank):
    c = _case(100 + R + V, R, K, V, rank, inputs.BF16)
    gu.say(f"ragged bf16 R={R} K={K} V={V} rank={rank}")
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    tok, lg, st = ch.run(want_logits=True)
    assert st == 0
    gu.assert_chain_parity(tok.cpu().numpy(), lg.cpu().numpy(), c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])


@pytest.mark.parametrize("R,K,V,rank", [(3, 5, 300, 7), (9, 2, 1025, 16), (1, 3, 64, 1)])
def test_ragged_fp32_parity(R, K, V, rank):
    c = _case(200 + R + V, R, K, V, rank, inputs.F32, base_std=1.0, factor_std=0.3)
    gu.say(f"ragged fp32 R={R} K={K} V={V} rank={rank}")
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.F32, c["prev0"])
    tok, lg, st = ch.run(want_logits=True)
    gu.assert_chain_parity(tok.cpu().numpy(), lg.cpu().numpy(), c["base"], c["A"], c["Bmat"], inputs.F32, c["prev0"])


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.F32])
def test_zero_bias_is_numpy_argmax_with_special_values(dtype):
    # Bmat = 0: the chain is numpy's argmax of each base row, NaN first, lowest index on ties.
    R, K, V, rank = 6, 3, 1536, 32
    rng = np.random.default_rng(9)
    x = rng.standard_normal((R, K, V)).astype(np.float32)
    x[0, 0, 700] = np.nan
    x[0, 0, 900] = np.nan
    x[1, 1, :] = -np.inf
    x[2, 2, 11] = np.inf
    x[2, 2, 12] = np.inf
    x[3, 0, :] = 0.0
    x[3, 0, 5] = -0.0
    x[4, 1, 1000] = x[4, 1].max() + 1
    x[4, 1, 3] = x[4, 1, 1000]          # exact tie: lower index wins
    x[5, 2, 1535] = 50.0                # last entry of the vocabulary
    if dtype == inputs.BF16:
        x = np.where(np.isnan(x), np.float32(np.nan), x)
        base = inputs.round_to_bf16(np.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0))
        base[np.isnan(x)] = 0x7FC0
        base[np.isposinf(x)] = 0x7F80
        base[np.isneginf(x)] = 0xFF80
        ref = inputs.bf16_to_f32(base)
    else:
        base, ref = x, x
    A = np.ones((V, rank), dtype=np.float32)
    Bmat = np.zeros((rank, V), dtype=np.float32)
    if dtype == inputs.BF16:
        A, Bmat = inputs.round_to_bf16(A), inputs.round_to_bf16(Bmat)
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    ch = gu.Chain(base, A, Bmat, dtype, prev0)
    tok, _, _ = ch.run()
    np.testing.assert_array_equal(tok.cpu().numpy(), np.argmax(ref, axis=2))


def test_closed_form_token_cycle_bf16():
    # A[v,:] = G e_{v mod r}, Bmat[k,v] = [v == k+1]: tok_i = (tok_{i-1} mod r) + 1 exactly.
    R, K, V, r, G = 20, 9, 3000, 64, 64.0
    rng = np.random.default_rng(3)
    base = inputs.round_to_bf16(rng.uniform(-1, 1, size=(R, K, V)).astype(np.float32))
    A = np.zeros((V, r), dtype=np.float32)
    A[np.arange(V), np.arange(V) % r] = G
    Bmat = np.zeros((r, V), dtype=np.float32)
    Bmat[np.arange(r), np.arange(r) + 1] = 1.0
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    ch = gu.Chain(base, inputs.round_to_bf16(A), inputs.round_to_bf16(Bmat), inputs.BF16, prev0)
    tok, _, _ = ch.run()
    tok = tok.cpu().numpy()
    for rr in range(R):
        p = prev0[rr]
        for i in range(K):
            p = (p % r) + 1
            assert tok[rr, i] == p, (rr, i)


def test_prev0_out_of_range_is_clamped_and_flagged():
    c = _case(5, 4, 2, 512, 32, inputs.BF16)
    bad = c["prev0"].copy()
    bad[0], bad[2] = -3, 512
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, bad)
    tok, _, st = ch.run()
    assert st == gu.B.STATUS_PREV_CLAMPED
    clamped = bad.copy()
    clamped[0], clamped[2] = 0, 511
    gu.assert_chain_parity(tok.cpu().numpy(), None, c["base"], c["A"], c["Bmat"], inputs.BF16, clamped)


def test_chain_is_deterministic():
    c = _case(6, 64, 5, 20000, 256, inputs.BF16)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    t1, l1, _ = ch.run(want_logits=True)
    t2, l2, _ = ch.run(want_logits=True)
    assert torch.equal(t1, t2)
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


# Without a logits output the chain runs the pipelined scorer (single launch when the
# requests fit one LDS chunk, one launch per position otherwise); these shapes cover
# partial ring cycles (R not a multiple of 64), the ragged last vocabulary tile, V not a
# multiple of 8, and request chunks that hand the base ring from one to the next.
@pytest.mark.parametrize("R,K,V,rank", [
    (5, 3, 1000, 64),
    (17, 2, 4104, 32),
    (33, 4, 777, 96),
    (64, 3, 5000, 256),
    (70, 5, 2600, 128),
    (250, 2, 3001, 256),
    (256, 4, 8192, 256),
    (300, 2, 2048, 256),
    (600, 2, 1544, 64),
    (1, 1, 1, 32),
])
def test_ragged_bf16_parity_fast_scorer(R, K, V, rank):
    c = _case(300 + R + V, R, K, V, rank, inputs.BF16)
    gu.say(f"fast scorer bf16 R={R} K={K} V={V} rank={rank}")
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    tok, _, st = ch.run()
    assert st == 0
    gu.assert_chain_parity(tok.cpu().numpy(), None, c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])


@pytest.mark.parametrize("R,V", [(70, 1000), (70, 1001), (130, 2048)])
def test_fast_scorer_special_values_match_numpy_argmax(R, V):
    # Bmat = 0 and bf16 inputs: every position is numpy's argmax of its base row.  NaNs,
    # infinities, signed zeros and exact ties sit in later request blocks and in the
    # ragged last tile, so the NaN rescore and the tail masking both run.
    K, rank = 3, 32
    rng = np.random.default_rng(R + V)
    x = rng.standard_normal((R, K, V)).astype(np.float32)
    x[65, 0, V - 1] = np.nan
    x[65, 0, 3] = np.nan
    x[66, 1, :] = -np.inf
    x[67, 2, V - 2] = np.inf
    x[67, 2, V - 1] = np.inf
    x[68, 0, :] = 0.0
    x[68, 0, 2] = -0.0
    x[69, 1, V - 1] = 40.0
    x[69, 1, V // 2] = 40.0
    x[1, 2, V - 1] = 30.0
    base = inputs.round_to_bf16(np.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0))
    base[np.isnan(x)] = 0x7FC0
    base[np.isposinf(x)] = 0x7F80
    base[np.isneginf(x)] = 0xFF80
    base[68, 0, 2] = 0x8000
    ref = inputs.bf16_to_f32(base)
    A = inputs.round_to_bf16(np.ones((V, rank), dtype=np.float32))
    Bmat = inputs.round_to_bf16(np.zeros((rank, V), dtype=np.float32))
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    ch = gu.Chain(base, A, Bmat, inputs.BF16, prev0)
    tok, _, _ = ch.run()
    np.testing.assert_array_equal(tok.cpu().numpy(), np.argmax(ref, axis=2))


# Vocabularies with more 512-entry tiles than the CUs hold at once (over 131072 entries on
# 256 CUs) and one request group (R <= 64) run two tiles per workgroup in one launch, the
# tile order flipping every position.  Shapes: ragged last tile, V not a multiple of 8, an
# odd tile count (the last workgroup's second tile is empty), ranks below 256.
@pytest.mark.parametrize("R,K,V,rank", [
    (40, 5, 140000, 256),
    (64, 4, 133635, 256),
    (7, 6, 131372, 128),
    (33, 3, 262144, 64),
])
def test_two_tile_chain_parity(R, K, V, rank):
    c = _case(400 + R + K, R, K, V, rank, inputs.BF16)
    gu.say(f"two-tile chain bf16 R={R} K={K} V={V} rank={rank}")
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    tok, _, st = ch.run()
    assert st == 0
    gu.assert_chain_parity(tok.cpu().numpy(), None, c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    tok2, _, _ = ch.run()
    assert torch.equal(tok, tok2)


def test_two_tile_chain_special_values_match_numpy_argmax():
    # Bmat = 0: every position is numpy's argmax of its base row; NaNs (the exact rescore),
    # infinities and ties sit in both tiles of a workgroup and in the empty-tile workgroup.
    R, K, V, rank = 10, 3, 131372, 32
    rng = np.random.default_rng(77)
    x = rng.standard_normal((R, K, V)).astype(np.float32)
    x[0, 0, 5] = np.nan
    x[0, 0, V - 1] = np.nan
    x[1, 1, 131000] = np.nan
    x[2, 2, :] = -np.inf
    x[3, 0, V - 2] = np.inf
    x[3, 0, V - 1] = np.inf
    x[4, 1, 200] = 40.0
    x[4, 1, 131100] = 40.0
    x[5, 2, 66000] = 30.0
    base = inputs.round_to_bf16(np.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0))
    base[np.isnan(x)] = 0x7FC0
    base[np.isposinf(x)] = 0x7F80
    base[np.isneginf(x)] = 0xFF80
    ref = inputs.bf16_to_f32(base)
    A = inputs.round_to_bf16(np.ones((V, rank), dtype=np.float32))
    Bmat = inputs.round_to_bf16(np.zeros((rank, V), dtype=np.float32))
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    ch = gu.Chain(base, A, Bmat, inputs.BF16, prev0)
    tok, _, _ = ch.run()
    np.testing.assert_array_equal(tok.cpu().numpy(), np.argmax(ref, axis=2))


def test_two_tile_chain_lds_slices_special_values():
    # Full rank, V a multiple of 8: the last waves of each workgroup score their second tile
    # from LDS.  Bmat = 0, so every position is numpy's argmax of its base row; NaNs (the
    # exact rescore from LDS), infinities and ties sit in those waves' vocabulary slices
    # (second tile b + G, G = 137 workgroups for V = 140000, wave offsets 320..511).
    R, K, V, rank = 10, 3, 140000, 256
    G = ((V + 511) // 512 + 1) // 2
    t2 = lambda b, off: (b + G) * 512 + off  # noqa: E731
    rng = np.random.default_rng(91)
    x = rng.standard_normal((R, K, V)).astype(np.float32)
    x[0, 0, t2(0, 400)] = np.nan
    x[0, 0, t2(5, 330)] = np.nan
    x[1, 1, t2(3, 511)] = np.inf
    x[1, 1, t2(2, 320)] = np.inf
    x[2, 2, t2(7, 350)] = 40.0
    x[2, 2, t2(1, 350)] = 40.0
    x[3, 0, :] = -np.inf
    x[4, 1, t2(135, 450)] = 35.0   # the last full second tile
    base = inputs.round_to_bf16(np.nan_to_num(x, nan=0.0, posinf=0.0, neginf=0.0))
    base[np.isnan(x)] = 0x7FC0
    base[np.isposinf(x)] = 0x7F80
    base[np.isneginf(x)] = 0xFF80
    ref = inputs.bf16_to_f32(base)
    A = inputs.round_to_bf16(np.ones((V, rank), dtype=np.float32))
    Bmat = inputs.round_to_bf16(np.zeros((rank, V), dtype=np.float32))
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    ch = gu.Chain(base, A, Bmat, inputs.BF16, prev0)
    tok, _, _ = ch.run()
    np.testing.assert_array_equal(tok.cpu().numpy(), np.argmax(ref, axis=2))
