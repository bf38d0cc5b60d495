"""GPU parity of dspark_step_sized: the budget sized from another (older) confidence
array and the first-drop admission rule, on the single-launch bf16 step and on the
stage-wise fp32 path, against the oracle's schedule with the same sizing array."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import inputs
from oracle import sched

pytestmark = pytest.mark.gpu

RULES = [B.RULE_ARGMAX, B.RULE_FIRST_DROP]


def _conf(w, seed, R=None):
    rng = np.random.default_rng(seed)
    conf = inputs._confidences(w, rng)
    if R == 0:
        return np.zeros((0, w.K), dtype=np.float32)
    if R is not None:
        reps = -(-R // conf.shape[0])
        conf = np.concatenate([conf] * reps)[:R].copy()
        conf[:, 0] = rng.uniform(0.3, 1.0, R).astype(np.float32)
    return conf


@pytest.mark.parametrize("name", ["small", "headline"])
@pytest.mark.parametrize("rule", RULES)
def test_stale_sized_step_matches_the_oracle(name, rule):
    w = inputs.WORKLOADS[name]
    gu.say(f"sized step {name} rule {rule}")
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    ref, _, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
    for size_R, seed in ((w.R, 11), (w.R // 2, 12), (w.R + w.R // 3, 13), (0, 14)):
        size_conf = _conf(w, seed, size_R)
        gu.say(f"  size_R={size_R}")
        got, status, _ = gu.run_step_sized(ch, ins.conf, size_conf, rule, w.n_sampling, w.T, w.R_all, vc, dc)
        assert status == 0
        np.testing.assert_array_equal(got["tokens"], ref["tokens"])   # the chain does not see the sizing
        want = sched.schedule(ins.conf, w.n_sampling, w.T, w.R_all, vc, dc, tokens=got["tokens"],
                              size_conf=size_conf, rule=rule)
        gu.assert_sched_parity(got, want, w.R, w.K)
    # no sizing array: the plain step under this rule
    got, _, _ = gu.run_step_sized(ch, ins.conf, None, rule, w.n_sampling, w.T, w.R_all, vc, dc)
    want = sched.schedule(ins.conf, w.n_sampling, w.T, w.R_all, vc, dc, tokens=got["tokens"], rule=rule)
    gu.assert_sched_parity(got, want, w.R, w.K)
    if rule == B.RULE_ARGMAX:
        for k in ref:
            assert np.array_equal(np.asarray(ref[k]), np.asarray(got[k])), k


@pytest.mark.parametrize("rule", RULES)
def test_stale_sized_step_on_the_stagewise_path(rule):
    # fp32 chains take the stage-wise launches (schedule kernel, chain kernels, finalize).
    w = inputs.WORKLOADS["tiny"]
    ins = inputs.generate(w)
    assert w.dtype == inputs.F32
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    for size_R, seed in ((w.R, 21), (1, 22), (3 * w.R, 23)):
        size_conf = _conf(w, seed, size_R)
        got, status, _ = gu.run_step_sized(ch, ins.conf, size_conf, rule, w.n_sampling, w.T, w.R_all, vc, dc)
        assert status == 0
        gu.assert_chain_parity(got["tokens"], None, ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
        want = sched.schedule(ins.conf, w.n_sampling, w.T, w.R_all, vc, dc, tokens=got["tokens"],
                              size_conf=size_conf, rule=rule)
        gu.assert_sched_parity(got, want, w.R, w.K)


def test_two_step_lag_over_a_sequence_of_steps():
    # A ring of three confidence buffers: step k sizes from step k-2's array (the first two
    # steps from the oldest one there is) and allocates from its own.
    w = inputs.WORKLOADS["small"]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    out = B.StepBuffers(w.R, w.K)
    confs = []
    for k in range(5):
        st = inputs.generate_step(w, k)
        confs.append(st["conf"])
        ch.base.copy_(gu.to_dev(st["base"]))
        ch.prev0.copy_(gu.to_dev(st["prev0"]))
        old = confs[max(0, k - 2)]
        got, status, _ = gu.run_step_sized(ch, st["conf"], old, B.RULE_ARGMAX, w.n_sampling, w.T, w.R_all, vc, dc,
                                           out=out)
        assert status == 0
        want = sched.schedule(st["conf"], w.n_sampling, w.T, w.R_all, vc, dc, tokens=got["tokens"], size_conf=old)
        gu.assert_sched_parity(got, want, w.R, w.K)


def test_one_workspace_serves_several_shapes():
    # The step's counters sit at a fixed place in the workspace, so one zero-filled
    # workspace sized for the largest shape serves smaller R and K in any order.
    w = inputs.WORKLOADS["headline"]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    big = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    ref_big, _, _ = gu.run_step(big, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
    shapes = [(100, 7), (256, 3), (7, 7), (256, 7), (33, 5)]
    refs = {}
    for R, K in shapes:   # each shape on a fresh workspace of its own
        sub = gu.Chain(ins.base[:R, :K].copy(), ins.A, ins.Bmat, w.dtype, ins.prev0[:R])
        refs[(R, K)] = gu.run_step(sub, ins.conf[:R, :K].copy(), w.n_sampling, w.T, w.R_all, vc, dc)[0]
        del sub
    for rep in range(2):
        for R, K in shapes:
            gu.say(f"shared workspace R={R} K={K} pass {rep}")
            sub = gu.Chain(ins.base[:R, :K].copy(), ins.A, ins.Bmat, w.dtype, ins.prev0[:R])
            sub.ws = big.ws
            got, st, _ = gu.run_step(sub, ins.conf[:R, :K].copy(), w.n_sampling, w.T, w.R_all, vc, dc)
            assert st == 0
            for k in got:
                assert np.array_equal(np.asarray(got[k]), np.asarray(refs[(R, K)][k])), (R, K, k)
            del sub
    again, _, _ = gu.run_step(big, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
    for k in again:
        assert np.array_equal(np.asarray(again[k]), np.asarray(ref_big[k])), k
