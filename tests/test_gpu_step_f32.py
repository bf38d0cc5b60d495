"""GPU parity of the whole step with fp32 factors.  Up to 64 requests it runs as one
launch (vocabulary workgroups plus the scheduling workgroup); above that, as the
per-position chain launches with the separate schedule launch.  Either way the tokens
must equal the per-position chain entry point's (same fp32 arithmetic), the chain must
match the fp64 oracle under the parity rules, and the schedule must match bit for bit."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import inputs
from oracle import sched

pytestmark = pytest.mark.gpu


def _tables(seed, n, R):
    rng = np.random.default_rng(seed)
    vc = np.maximum.accumulate(100.0 + 0.5 * np.arange(n + 65) + rng.normal(0, 0.3, n + 65)).astype(np.float32)
    dc = np.maximum.accumulate(10.0 + 0.2 * np.arange(R + 1)).astype(np.float32)
    return vc, dc


def _check(c, R, K, got, status, ch, vc, dc, expect_status=0):
    assert status == expect_status, status
    gu.assert_chain_parity(got["tokens"], None, c["base"], c["A"], c["Bmat"], inputs.F32, c["prev0"])
    tok, _, _ = ch.run()
    np.testing.assert_array_equal(tok.cpu().numpy(), got["tokens"])
    want = sched.schedule(c["conf"], R, 0, R, vc, dc, tokens=got["tokens"])
    gu.assert_sched_parity(got, want, R, K)


# (R, K, V, rank): the whole vocabulary in one chain workgroup (V <= 2048, rank <= 16),
# several workgroups (rank <= 16 and rank <= 64 forms), ragged V, rank 1 .. 100, the
# single-launch limits (64 requests, rank 64) and past them (per-position launches)
CASES = [(1, 3, 700, 5), (4, 7, 1024, 16), (64, 2, 513, 1), (3, 5, 2048, 16), (9, 4, 5000, 12),
         (17, 5, 1531, 33), (40, 9, 4099, 64), (64, 7, 2048, 100), (65, 4, 1500, 16)]


@pytest.mark.parametrize("R,K,V,rank", CASES)
def test_f32_step_parity(R, K, V, rank):
    gu.say(f"f32 step R={R} K={K} V={V} rank={rank}")
    c = inputs.random_case(500 + R + V, R=R, K=K, V=V, rank=rank, dtype=inputs.F32)
    vc, dc = _tables(R * K, R * K, R)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.F32, c["prev0"])
    got, status, _ = gu.run_step(ch, c["conf"], R, 0, R, vc, dc)
    _check(c, R, K, got, status, ch, vc, dc)


def test_f32_step_clamps_prev0_and_reports_it():
    R, K, V, rank = 6, 4, 900, 8
    c = inputs.random_case(91, R=R, K=K, V=V, rank=rank, dtype=inputs.F32)
    c["prev0"][1] = -3
    c["prev0"][4] = V + 5
    vc, dc = _tables(3, R * K, R)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.F32, c["prev0"])
    got, status, _ = gu.run_step(ch, c["conf"], R, 0, R, vc, dc)
    _check(c, R, K, got, status, ch, vc, dc, expect_status=B.STATUS_PREV_CLAMPED)


def test_f32_step_repeats_and_interleaves_on_one_workspace():
    # The scheduling workgroup puts the barrier counters and the ready flag back to zero at
    # the end of each launch; the per-position chain entry point zeroes its own region.
    R, K, V, rank = 8, 7, 1100, 16
    c = inputs.random_case(17, R=R, K=K, V=V, rank=rank, dtype=inputs.F32)
    vc, dc = _tables(5, R * K, R)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.F32, c["prev0"])
    first, st, _ = gu.run_step(ch, c["conf"], R, 0, R, vc, dc)
    assert st == 0
    for rep in range(3):
        tok, _, st = ch.run()
        assert st == 0
        np.testing.assert_array_equal(tok.cpu().numpy(), first["tokens"])
        for _ in range(2):
            got, st, _ = gu.run_step(ch, c["conf"], R, 0, R, vc, dc)
            assert st == 0
            for k in first:
                assert np.array_equal(np.asarray(first[k]), np.asarray(got[k])), (rep, k)


def test_f32_step_launch_modes_agree():
    R, K, V, rank = 4, 7, 1024, 16
    c = inputs.random_case(23, R=R, K=K, V=V, rank=rank, dtype=inputs.F32)
    vc, dc = _tables(7, R * K, R)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.F32, c["prev0"])
    res, st_r, _ = gu.run_step(ch, c["conf"], R, 0, R, vc, dc)
    try:
        B.dspark_set_launch_mode(B.LAUNCH_COOPERATIVE)
        coop, st_c, _ = gu.run_step(ch, c["conf"], R, 0, R, vc, dc)
    finally:
        B.dspark_set_launch_mode(B.LAUNCH_RESIDENT)
    assert st_r == st_c == 0
    for k in res:
        assert np.array_equal(np.asarray(res[k]), np.asarray(coop[k])), k
