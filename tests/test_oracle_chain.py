"""Pins of the chain oracle (stage 1) against things other than itself.

Each pin is chosen so that a plausible slip in the oracle -- a dropped base or
bias term, a transposed factor, the wrong previous token, a wrong sign, a
NaN-unsafe argmax -- fails at least one test.
"""
import numpy as np
import pytest

import oracle
from confidence_scheduled_verification_amd import inputs


def _f32_case(seed, R, K, V, rank, base_std=1.0, fstd=0.1):
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((R, K, V)).astype(np.float32) * np.float32(base_std)
    A = rng.standard_normal((V, rank)).astype(np.float32) * np.float32(fstd)
    Bmat = rng.standard_normal((rank, V)).astype(np.float32) * np.float32(fstd)
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    return base, A, Bmat, prev0


def test_zero_bias_is_plain_argmax():
    # Special case Bmat = 0: every position is numpy's argmax of its base row, whatever prev is.
    base, A, _, prev0 = _f32_case(1, R=5, K=4, V=300, rank=8)
    base[1, 2, 17] = np.nan             # numpy's argmax returns the first NaN
    base[1, 2, 200] = np.nan
    base[3, 1, :] = -np.inf             # all -inf: index 0
    base[4, 0, 5] = np.inf
    Bmat = np.zeros((8, 300), dtype=np.float32)
    tok, _, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0)
    np.testing.assert_array_equal(tok, np.argmax(base, axis=2))
    assert tok[1, 2] == 17 and tok[3, 1] == 0 and tok[4, 0] == 5


def test_closed_form_cycle():
    # A[v,:] = G e_{v mod r}, Bmat[k,v] = [v == k+1]  =>  W[u,v] = G [v == (u mod r) + 1],
    # so with |base| << G the chain follows tok_i = (tok_{i-1} mod r) + 1.
    # A transposed factor, a wrong prev or a dropped bias breaks the cycle.
    R, K, V, r, G = 6, 9, 50, 8, 100.0
    rng = np.random.default_rng(2)
    base = (rng.uniform(-1, 1, size=(R, K, V))).astype(np.float32)
    A = np.zeros((V, r), dtype=np.float32)
    A[np.arange(V), np.arange(V) % r] = G
    Bmat = np.zeros((r, V), dtype=np.float32)
    Bmat[np.arange(r), np.arange(r) + 1] = 1.0
    prev0 = rng.integers(0, V, size=R, dtype=np.int32)
    tok, _, st = oracle.chain(base, A, Bmat, inputs.F32, prev0)
    assert st == 0
    for rr in range(R):
        p = prev0[rr]
        for i in range(K):
            p = (p % r) + 1
            assert tok[rr, i] == p


def test_single_position_matches_numpy_matmul():
    # K = 1: x = base + A[prev0] @ Bmat, computed by numpy's float64 matmul.
    base, A, Bmat, prev0 = _f32_case(3, R=7, K=1, V=513, rank=24)
    tok, logits, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0, want_logits=True)
    ref = base[:, 0, :].astype(np.float64) + A[prev0].astype(np.float64) @ Bmat.astype(np.float64)
    np.testing.assert_allclose(logits[:, 0, :], ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(tok[:, 0], np.argmax(ref, axis=1))


def test_multi_position_matches_numpy_stepwise():
    # Every position equals numpy's matmul keyed on the oracle's own previous token.
    base, A, Bmat, prev0 = _f32_case(4, R=3, K=6, V=257, rank=16, base_std=0.05, fstd=0.5)
    tok, logits, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0, want_logits=True)
    prev = prev0.copy()
    changed = 0
    for i in range(6):
        ref = base[:, i, :].astype(np.float64) + A[prev].astype(np.float64) @ Bmat.astype(np.float64)
        np.testing.assert_allclose(logits[:, i, :], ref, rtol=1e-12, atol=1e-12)
        t = np.argmax(ref, axis=1)
        changed += int(np.sum(t != np.argmax(base[:, i, :], axis=1)))
        np.testing.assert_array_equal(tok[:, i], t)
        prev = t.astype(np.int32)
    assert changed > 0   # the bias really moves the argmax in this case


def test_bf16_inputs_widen_exactly():
    w = inputs.WORKLOADS["small"]
    case = inputs.random_case(5, R=2, K=3, V=96, rank=32, dtype=inputs.BF16)
    tok, logits, _ = oracle.chain(case["base"], case["A"], case["Bmat"], inputs.BF16, case["prev0"],
                                  want_logits=True)
    base = inputs.bf16_to_f32(case["base"]).astype(np.float64)
    A = inputs.bf16_to_f32(case["A"]).astype(np.float64)
    Bm = inputs.bf16_to_f32(case["Bmat"]).astype(np.float64)
    prev = case["prev0"]
    for i in range(3):
        ref = base[:, i, :] + A[prev] @ Bm
        np.testing.assert_allclose(logits[:, i, :], ref, rtol=1e-13, atol=1e-13)
        prev = tok[:, i]
    assert w.dtype == inputs.BF16


def test_teacher_forcing_with_own_tokens_is_identity():
    base, A, Bmat, prev0 = _f32_case(6, R=4, K=5, V=200, rank=8)
    tok, lg, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0, want_logits=True)
    tok2, lg2, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0, forced=tok, want_logits=True)
    np.testing.assert_array_equal(tok, tok2)
    np.testing.assert_array_equal(lg, lg2)


def test_teacher_forcing_keys_on_forced_token():
    base, A, Bmat, prev0 = _f32_case(7, R=2, K=3, V=64, rank=8, base_std=0.01, fstd=1.0)
    forced = np.array([[5, 9, 0], [63, 1, 0]], dtype=np.int32)
    tok, lg, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0, forced=forced, want_logits=True)
    for r in range(2):
        for i in (1, 2):
            ref = base[r, i].astype(np.float64) + A[forced[r, i - 1]].astype(np.float64) @ Bmat.astype(np.float64)
            np.testing.assert_allclose(lg[r, i], ref, rtol=1e-13, atol=1e-13)


def test_row_subset_equals_full_run():
    base, A, Bmat, prev0 = _f32_case(8, R=6, K=3, V=100, rank=8)
    full, _, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0)
    sub, _, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0, rows=[4, 1])
    np.testing.assert_array_equal(sub, full[[4, 1]])


def test_prev0_out_of_range_is_clamped():
    base, A, Bmat, prev0 = _f32_case(9, R=3, K=2, V=50, rank=4)
    bad = np.array([-7, 50, 3], dtype=np.int32)
    tok, _, st = oracle.chain(base, A, Bmat, inputs.F32, bad)
    ok = np.array([0, 49, 3], dtype=np.int32)
    tok2, _, st2 = oracle.chain(base, A, Bmat, inputs.F32, ok)
    np.testing.assert_array_equal(tok, tok2)
    assert st == 1 and st2 == 0


def test_nan_in_factor_row_gives_nan_winner_first_index():
    # A NaN in the keyed factor row makes every logit NaN: the first index (0) wins.
    base, A, Bmat, prev0 = _f32_case(10, R=1, K=2, V=40, rank=4)
    prev0[:] = 3
    A[3, 1] = np.nan
    tok, _, _ = oracle.chain(base, A, Bmat, inputs.F32, prev0)
    assert tok[0, 0] == 0
