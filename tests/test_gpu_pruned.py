"""GPU parity of the pruned chain (stage 1 scored over the candidates its bias bound
leaves, cand_chain_kernel) where the pruning itself could go wrong: rows the bound cannot
prune (the dense fallback), a bound that is not finite, special values under a live
bias, guessed key rows that miss, ragged vocabularies and the limits of the form.  Every
row is compared with the teacher-forced oracle, and with the dense form on the same
inputs (the two forms may differ only at float32 near-ties)."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import inputs

pytestmark = pytest.mark.gpu


def _both_forms(c, R, K, V, rank, dtype=inputs.BF16):
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], dtype, c["prev0"])
    with gu.chain_form(B.CHAIN_PRUNED):
        tp, _, sp = ch.run()
        tp2, _, _ = ch.run()
    with gu.chain_form(B.CHAIN_DENSE):
        td, _, sd = ch.run()
    tp, tp2, td = tp.cpu().numpy(), tp2.cpu().numpy(), td.cpu().numpy()
    np.testing.assert_array_equal(tp, tp2)  # the pruned form is deterministic
    near = gu.assert_chain_parity(tp, None, c["base"], c["A"], c["Bmat"], dtype, c["prev0"])
    gu.assert_tokens_agree(tp, td, c["base"], c["A"], c["Bmat"], dtype, c["prev0"])
    return tp, sp, sd, near


def _case(seed, R, K, V, rank, base_std=2.0, factor_std=0.05):
    rng = np.random.default_rng(seed)
    base = inputs.round_to_bf16(rng.standard_normal((R, K, V), dtype=np.float32) * base_std)
    A = inputs.round_to_bf16(rng.standard_normal((V, rank), dtype=np.float32) * factor_std)
    Bmat = inputs.round_to_bf16(rng.standard_normal((rank, V), dtype=np.float32) * factor_std)
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    return {"base": base, "A": A, "Bmat": Bmat, "prev0": prev0}


@pytest.mark.parametrize("R,K,V,rank,factor_std", [
    (6, 3, 20000, 64, 1.0),      # bias far above the logits' spread: every entry a candidate
    (5, 4, 9000, 256, 0.2),      # candidates past the per-row share of the list
    (2, 32, 5000, 64, 1.0),      # more kept groups than the LDS pool holds
    (1, 2, 70000, 32, 1.0),      # one row's kept groups past the chunk table
])
def test_rows_the_bound_cannot_prune_are_scored_densely(R, K, V, rank, factor_std):
    gu.say(f"weak bound R={R} K={K} V={V} rank={rank} factor_std={factor_std}")
    c = _case(1000 + V, R, K, V, rank, base_std=0.5, factor_std=factor_std)
    _, sp, sd, _ = _both_forms(c, R, K, V, rank)
    assert sp == sd == 0


def test_non_finite_bound_scores_every_row_densely():
    # an infinite entry in A makes the bound infinite: every row is scored over the whole
    # vocabulary, with IEEE propagation wherever that row of A is the key
    R, K, V, rank = 4, 3, 6000, 32
    c = _case(77, R, K, V, rank)
    c["A"][V - 1, 5] = np.uint16(0x7F80)  # +inf in the row of token V-1
    c["prev0"][0] = V - 1                  # request 0 starts keyed on it
    _both_forms(c, R, K, V, rank)


def test_special_values_with_a_live_bias():
    # NaN rows (first NaN wins), a -inf row (token 0), +inf entries (the first +inf wins),
    # ties at the maximum, in several items of a row, with a bias that is not zero
    R, K, V, rank = 6, 4, 14000, 64
    c = _case(5, R, K, V, rank)
    b = c["base"]
    nan, pinf, ninf = np.uint16(0x7FC0), np.uint16(0x7F80), np.uint16(0xFF80)
    b[0, 1, 9000] = nan
    b[0, 1, 12000] = nan
    b[1, 0, :] = ninf
    b[2, 2, 5000] = pinf
    b[2, 2, 13999] = pinf
    b[3, 3, 4095] = nan                         # item boundary
    b[3, 3, 4096] = pinf
    top = np.uint16(0x4170)                     # 15.0 in bf16: far above the rest of the row
    b[4, 0, 100] = top
    b[4, 0, 8191] = top                         # a tie at the maximum in another item
    b[5, 1, :] = nan                            # a row of NaN: index 0
    tp, sp, _, _ = _both_forms(c, R, K, V, rank)
    assert sp == 0
    assert tp[0, 1] == 9000 and tp[1, 0] == 0 and tp[2, 2] == 5000 and tp[3, 3] == 4095 and tp[5, 1] == 0


@pytest.mark.parametrize("seed", [3, 4])
def test_guessed_key_rows_that_miss(seed):
    # a bias large enough to reorder the top of many rows, with a bound that still prunes:
    # the key row guessed for position i+1 (row i's largest logit) is wrong wherever row
    # i's token is not its largest logit, and position i+1 is then scored again
    R, K, V, rank = 24, 4, 10000, 256
    c = _case(seed, R, K, V, rank, base_std=2.0, factor_std=0.07)
    tp, _, _, _ = _both_forms(c, R, K, V, rank)
    base = inputs.bf16_to_f32(c["base"])
    top = np.argmax(base, axis=2)
    misses = int(np.sum(tp[:, :-1] != top[:, :-1]))
    gu.say(f"guessed key rows missed at {misses} of {R * (K - 1)} positions")
    assert misses > 0


@pytest.mark.parametrize("R,K,V,rank", [
    (3, 32, 5000, 64),          # the pruned form's K limit
    (3, 33, 5000, 64),          # past it: the dense form
    (2, 2, 262144, 32),         # the pruned form's V limit
    (2, 2, 262152, 32),         # past it
    (5, 3, 10001, 96),          # V not a multiple of 8 (element-wise loads)
    (4, 2, 4095, 32),           # one item per row, ragged
    (3, 2, 1, 32),              # a single-entry vocabulary
    (1, 1, 4096, 256),          # one item exactly
])
def test_pruned_form_shapes(R, K, V, rank):
    gu.say(f"pruned shapes R={R} K={K} V={V} rank={rank}")
    c = _case(R * 1000 + K * 10 + V % 97, R, K, V, rank)
    _, sp, sd, _ = _both_forms(c, R, K, V, rank)
    assert sp == sd == 0


def test_pruned_step_matches_the_oracle_on_a_fresh_draw_each_step():
    # the counters a chain leaves for the next launch are back at zero after every step,
    # whatever the shape: one workspace, four steps of two shapes
    w = inputs.WORKLOADS["small"]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    for k in range(4):
        st = inputs.generate_step(w, k)
        R = w.R if k % 2 == 0 else w.R // 2
        base, prev0, conf = st["base"][:R], st["prev0"][:R], st["conf"][:R]
        sub = gu.Chain.__new__(gu.Chain)
        sub.__dict__.update(ch.__dict__)
        sub.R = R
        sub.base = gu.to_dev(base)
        sub.prev0 = gu.to_dev(prev0)
        got, status, _ = gu.run_step(sub, conf, R, w.T, R, vc, dc)
        assert status == 0
        gu.assert_chain_parity(got["tokens"], None, base, ins.A, ins.Bmat, w.dtype, prev0)


def test_winner_at_the_edge_of_the_key_row_bound():
    # Position 0 of request 0 is keyed on a row of A whose norm is well below A's largest,
    # so the chain's floor uses the key row's own norm.  The winner's Bt row points along
    # the key row and the row maximum's against it: the winner's logit lies 2|a||b| below
    # the maximum plus 0.03, just inside that floor, and only its exact score finds it.
    R, K, V, rank = 2, 2, 5000, 64
    c = _case(4242, R, K, V, rank, base_std=0.3, factor_std=0.02)
    rng = np.random.default_rng(4243)
    p, u_top, v_win, b = 7, 100, 200, 0.5
    key = rng.standard_normal(rank).astype(np.float32)
    key *= 0.5 / np.linalg.norm(key)
    A_f = rng.standard_normal((V, rank)).astype(np.float32) * 0.125  # other rows: norm about 1
    A_f[p] = key
    c["A"] = inputs.round_to_bf16(A_f)
    unit = key / np.linalg.norm(key)
    Bm = (rng.standard_normal((rank, V)).astype(np.float32) * 0.02)
    Bm[:, v_win] = b * unit
    Bm[:, u_top] = -b * unit
    c["Bmat"] = inputs.round_to_bf16(Bm)
    c["prev0"][0] = p
    # the exact biases of the two rows from the bf16 values, and the base logits around them
    a16 = c["A"].astype(np.uint32) << 16
    m16 = c["Bmat"].astype(np.uint32) << 16
    a_row = a16[p].view(np.float32).astype(np.float64)
    bias = lambda v: float(a_row @ m16[:, v].view(np.float32).astype(np.float64))
    top = 4.0
    base = (c["base"].astype(np.uint32) << 16).view(np.float32)
    base[0, 0, u_top] = top
    base[0, 0, v_win] = top + bias(u_top) - bias(v_win) + 0.03
    c["base"] = inputs.round_to_bf16(base)
    tp, sp, sd, _ = _both_forms(c, R, K, V, rank)
    assert sp == sd == 0
    assert tp[0, 0] == v_win


@pytest.mark.parametrize("R,K,V,rank", [
    (8, 5, 30000, 64),     # 4 workgroups per request
    (100, 3, 20000, 256),  # 2 per request
    (3, 7, 9000, 32),      # 2 per request over 3 items a row, the fewest a split allows
])
def test_split_requests_match_one_workgroup_per_request(R, K, V, rank):
    # With fewer requests than compute units each request is streamed by several
    # workgroups whose helpers hand their kept groups to the owner through the workspace.
    # A workspace without room for those groups keeps one workgroup per request: both
    # must give the oracle's tokens, and the same ones (the argmax is unique here).
    gu.say(f"split vs whole requests R={R} K={K} V={V} rank={rank}")
    c = _case(77 + R * 13 + V % 101, R, K, V, rank)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    split, _, st_split = ch.run()
    small = B.workspace(256, K, V, rank, inputs.BF16)  # the minimum at R <= 256: no room for the split
    assert small.numel() * 8 < B.dspark_workspace_bytes(R, K, V, rank, inputs.BF16)
    ch.ws = small
    whole, _, st_whole = ch.run()
    assert st_split == st_whole == 0
    split, whole = split.cpu().numpy(), whole.cpu().numpy()
    gu.assert_chain_parity(split, None, c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    np.testing.assert_array_equal(split, whole)
