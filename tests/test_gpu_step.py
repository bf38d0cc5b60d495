"""GPU parity of the fused step (dspark_step) on every workload at its full size,
in the launch configuration the benchmark times.  Every chain row's tokens are
compared with the teacher-forced fp64 oracle (rows split over host threads) and the
schedule in full; the debug logits output is checked on a few rows."""
import dataclasses

import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import inputs
from oracle import sched

pytestmark = pytest.mark.gpu

# rows whose float32 chained logits (the debug output of the stage-1 entry point) are
# compared within the logit tolerance; tokens are compared on every row
LOGIT_ROWS = {"tiny": None, "small": None, "mid": [0, 37, 111], "headline": [0, 101, 255],
              "large": [0, 63]}


@pytest.mark.parametrize("form", ["pruned", "dense"])
@pytest.mark.parametrize("name", ["tiny", "small", "mid", "headline", "large"])
def test_full_size_step_parity(name, form):
    w = inputs.WORKLOADS[name]
    with gu.chain_form(gu.FORMS[form]):
        _full_size_step_parity(w, name)


def _full_size_step_parity(w, name):
    gu.say(f"step {name}: generating R={w.R} K={w.K} V={w.V}")
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    gu.say(f"step {name}: running")
    got, status, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
    assert status == 0
    gu.say(f"step {name}: oracle on all {w.R} rows")
    near = gu.assert_chain_parity(got["tokens"], None, ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    gu.say(f"step {name}: tokens ok on every row ({near} near-ties)")
    rows = LOGIT_ROWS[name]
    want = sched.schedule(ins.conf, w.n_sampling, w.T, w.R_all, vc, dc, tokens=got["tokens"])
    gu.assert_sched_parity(got, want, w.R, w.K)
    # the chained logits of the sampled rows, from the stage-1 entry point on the same inputs
    # (the dense form: asking for logits selects it); its tokens agree up to near-ties
    tok, lg, _ = ch.run(want_logits=True)
    gu.assert_tokens_agree(got["tokens"], tok.cpu().numpy(), ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    sel = np.arange(w.R) if rows is None else np.array(rows)
    gu.assert_chain_parity(tok.cpu().numpy(), lg[torch.as_tensor(sel, device=gu.DEV)].cpu().numpy(), ins.base, ins.A,
                           ins.Bmat, w.dtype, ins.prev0, rows=sel)


def test_step_is_deterministic_and_equals_stagewise():
    w = inputs.WORKLOADS["headline"]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    a, _, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
    b, _, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
    tok, _, _ = ch.run()
    np.testing.assert_array_equal(tok.cpu().numpy(), a["tokens"])
    R, K = w.R, w.K
    assert np.array_equal(a["ver_tokens"][:a["b_star"]], a["tokens"].reshape(-1)[a["ver_idx"][:a["b_star"]]])
    assert np.all(a["ver_tokens"][a["b_star"]:] == -1)


@pytest.mark.parametrize("name,form", [("mid", "pruned"), ("headline", "pruned"), ("headline", "dense")])
def test_timing_events_leave_the_step_unchanged(name, form):
    # With timing events set, the pruned chain's launch carries them (they take the kernel's
    # own start and stop; Mid splits its requests, the Headline does not) and the dense form
    # records them as markers: the step's results are the same as without, and the events
    # bracket a positive time.
    w = inputs.WORKLOADS[name]
    gu.say(f"timing events {name} {form}")
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    with gu.chain_form(gu.FORMS[form]):
        ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
        a, sa, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
        e1, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e1.record()
        e2.record()  # the HIP events exist before the library sets them
        torch.cuda.synchronize()
        B.dspark_set_timing_events(e1, e2)
        try:
            b, sb, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
        finally:
            B.dspark_set_timing_events(None, None)
    assert sa == sb == 0
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
    ms = e1.elapsed_time(e2)
    assert 0.0 < ms < 1000.0, ms


def test_multi_step_inputs_change_the_result():
    w = inputs.WORKLOADS["small"]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    out = B.StepBuffers(w.R, w.K)
    for k in range(3):
        st = inputs.generate_step(w, k)
        ch.base.copy_(gu.to_dev(st["base"]))
        ch.prev0.copy_(gu.to_dev(st["prev0"]))
        got, _, _ = gu.run_step(ch, st["conf"], w.n_sampling, w.T, w.R_all, vc, dc, out=out)
        gu.assert_chain_parity(got["tokens"], None, st["base"], ins.A, ins.Bmat, w.dtype, st["prev0"])
        want = sched.schedule(st["conf"], w.n_sampling, w.T, w.R_all, vc, dc, tokens=got["tokens"])
        gu.assert_sched_parity(got, want, w.R, w.K)


def test_empty_batch_step():
    w = inputs.WORKLOADS["tiny"]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    base = np.zeros((0, w.K, w.V), dtype=np.float32)
    ch = gu.Chain(base, ins.A, ins.Bmat, w.dtype, np.zeros(0, np.int32))
    got, status, _ = gu.run_step(ch, np.zeros((0, w.K), np.float32), 0, 0, 0, vc, dc)
    assert got["b_star"] == 0 and got["offsets"].tolist() == [0]
    assert got["best_obj"] == 0.0 and status == 0


def test_single_launch_step_keeps_the_workspace_consistent():
    # The single-launch step zeroes its keys in-launch and leaves its barrier counters
    # and ready flag at zero; the stage-wise chain zeroes the whole workspace first.
    # Interleaving them on one workspace must not change any result.
    w = inputs.WORKLOADS["small"]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    first, st0, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
    assert st0 == 0
    for rep in range(4):
        gu.say(f"workspace reuse round {rep}")
        tok, _, st = ch.run()
        assert st == 0
        np.testing.assert_array_equal(tok.cpu().numpy(), first["tokens"])
        for _ in range(2):
            got, st, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
            assert st == 0
            for k in first:
                assert np.array_equal(np.asarray(first[k]), np.asarray(got[k])), (rep, k)


def test_single_launch_step_at_the_slot_limit():
    # R = 256 requests x K = 64 positions = 16384 slots, the scheduler's maximum, inside
    # the single launch (its scheduling workgroup has 512 threads).
    R, K, V, rank = 256, 64, 2048, 32
    c = inputs.random_case(77, R=R, K=K, V=V, rank=rank, dtype=inputs.BF16)
    rng = np.random.default_rng(5)
    conf = rng.beta(4.0, 1.5, size=(R, K)).astype(np.float32)
    conf[rng.random((R, K)) < 0.02] = 1.0
    w = inputs.WORKLOADS["headline"]
    vlen = R * K + 64
    vc = np.maximum.accumulate(50.0 + 0.01 * np.arange(vlen) + rng.normal(0, 0.5, vlen)).astype(np.float32)
    dc = np.maximum.accumulate(5.0 + 0.1 * np.arange(R + 1)).astype(np.float32)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    got, status, _ = gu.run_step(ch, conf, R, 0, R, vc, dc)
    assert status == 0
    gu.assert_chain_parity(got["tokens"], None, c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    want = sched.schedule(conf, R, 0, R, vc, dc, tokens=got["tokens"])
    gu.assert_sched_parity(got, want, R, K)
    assert 0 < got["b_star"] < R * K


@pytest.mark.parametrize("name", ["small", "headline", "large"])
def test_launch_modes_give_identical_results(name):
    # The dense form's persistent kernels run as a plain launch of a resident grid
    # (default) or as a cooperative launch; the work is the same, so every output must
    # match bit for bit.  Large runs the two-tile chain beside a separate schedule launch.
    with gu.chain_form(B.CHAIN_DENSE):
        _launch_modes(name)


def _launch_modes(name):
    w = inputs.WORKLOADS[name]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    assert B.dspark_get_launch_mode() == B.LAUNCH_RESIDENT
    res, st_r, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
    tok_r, _, st_cr = ch.run()
    try:
        B.dspark_set_launch_mode(B.LAUNCH_COOPERATIVE)
        coop, st_c, _ = gu.run_step(ch, ins.conf, w.n_sampling, w.T, w.R_all, vc, dc)
        tok_c, _, st_cc = ch.run()
    finally:
        B.dspark_set_launch_mode(B.LAUNCH_RESIDENT)
    assert st_r == st_c == st_cr == st_cc == 0
    for k in res:
        assert np.array_equal(np.asarray(res[k]), np.asarray(coop[k])), k
    np.testing.assert_array_equal(tok_r.cpu().numpy(), tok_c.cpu().numpy())
    np.testing.assert_array_equal(tok_r.cpu().numpy(), res["tokens"])


@pytest.mark.parametrize("form", ["pruned", "dense"])
@pytest.mark.parametrize("R", [1, 17, 33, 64, 65])
def test_ring_depth_boundaries(R, form):
    with gu.chain_form(gu.FORMS[form]):
        _ring_depth(R)


def _ring_depth(R):
    # Up to 64 requests at the full rank the chain sweeps 2-block base rings (one group);
    # from 65 on, 4-block rings in two groups.  Both must give the oracle's tokens, the same
    # tokens through the step and the chain entry point, and the oracle's schedule.
    K, V, rank = 3, 3001, 256
    c = inputs.random_case(900 + R, R=R, K=K, V=V, rank=rank, dtype=inputs.BF16)
    rng = np.random.default_rng(R)
    vc = np.maximum.accumulate(80.0 + 0.7 * np.arange(R * K + 64) + rng.normal(0, 0.4, R * K + 64)).astype(np.float32)
    dc = np.maximum.accumulate(9.0 + 0.3 * np.arange(R + 1)).astype(np.float32)
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    got, status, _ = gu.run_step(ch, c["conf"], R, 0, R, vc, dc)
    assert status == 0
    gu.assert_chain_parity(got["tokens"], None, c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    tok, _, st = ch.run()
    assert st == 0
    np.testing.assert_array_equal(tok.cpu().numpy(), got["tokens"])
    want = sched.schedule(c["conf"], R, 0, R, vc, dc, tokens=got["tokens"])
    gu.assert_sched_parity(got, want, R, K)


# Vocabulary sizes on the boundaries between the step's launch forms (256 compute units,
# 512-entry tiles): 255 tiles take the single launch with its scheduling workgroup; 256
# tiles, the schedule launch and the single-launch chain; 257 tiles with R <= 64, the
# two-tile chain; 514 tiles, one chain launch per position.  Every form must give the
# oracle's tokens and schedule.
@pytest.mark.parametrize("form", ["pruned", "dense"])
@pytest.mark.parametrize("R,K,V,rank", [
    (16, 3, 255 * 512, 256),
    (16, 3, 255 * 512 + 8, 256),
    (16, 3, 256 * 512 + 8, 256),
    (8, 2, 514 * 512 - 40, 64),
])
def test_step_launch_form_boundaries(R, K, V, rank, form):
    with gu.chain_form(gu.FORMS[form]):
        _launch_form_boundary(R, K, V, rank)


def _launch_form_boundary(R, K, V, rank):
    c = inputs.random_case(700 + V % 97, R=R, K=K, V=V, rank=rank, dtype=inputs.BF16)
    w = dataclasses.replace(inputs.WORKLOADS["small"], R=R, R_all=R, K=K, V=V, rank=rank, n_sampling=R)
    vc = sched.force_monotone(inputs.raw_verify_cost(w, None))
    dc = sched.force_monotone(inputs.raw_draft_cost(w))
    gu.say(f"launch-form boundary R={R} K={K} V={V} rank={rank}")
    ch = gu.Chain(c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    got, status, _ = gu.run_step(ch, c["conf"], R, 0, R, vc, dc)
    assert status == 0
    gu.assert_chain_parity(got["tokens"], None, c["base"], c["A"], c["Bmat"], inputs.BF16, c["prev0"])
    want = sched.schedule(c["conf"], R, 0, R, vc, dc, tokens=got["tokens"])
    gu.assert_sched_parity(got, want, R, K)
    tok, _, _ = ch.run()
    np.testing.assert_array_equal(tok.cpu().numpy(), got["tokens"])
