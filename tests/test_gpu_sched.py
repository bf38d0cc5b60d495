"""GPU parity of stages 2-5 (survival, top-B, budget, allocation) against the oracle.

Every comparison is bit-exact: survivals, ranking, sorted survivals, B*, the
objective (both sides round the exact sum once), prefix lengths, offsets and
the compacted lists."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import inputs
from oracle import sched

pytestmark = pytest.mark.gpu


def _stagewise(conf, n_sampling, T, num_reqs, vc, dc, tokens=None):
    """Run the four stage entry points one after another on the GPU."""
    R, K = conf.shape
    n = R * K
    conf_d = gu.to_dev(conf.astype(np.float32))
    surv = torch.empty((R, K), dtype=torch.float32, device=gu.DEV)
    order = torch.empty(n, dtype=torch.int32, device=gu.DEV)
    ss = torch.empty(n, dtype=torch.float32, device=gu.DEV)
    rank = torch.empty(n, dtype=torch.int32, device=gu.DEV)
    b_star = torch.empty(1, dtype=torch.int32, device=gu.DEV)
    best = torch.empty(1, dtype=torch.float64, device=gu.DEV)
    bmax = min(n, len(vc) - 1 - T)
    obj = torch.empty(bmax + 1, dtype=torch.float64, device=gu.DEV)
    pl = torch.empty(R, dtype=torch.int32, device=gu.DEV)
    off = torch.empty(R + 1, dtype=torch.int32, device=gu.DEV)
    vi = torch.empty(n, dtype=torch.int32, device=gu.DEV)
    vt = torch.empty(n, dtype=torch.int32, device=gu.DEV) if tokens is not None else None
    tok_d = gu.to_dev(tokens.astype(np.int32)) if tokens is not None else None
    status = torch.zeros(1, dtype=torch.int32, device=gu.DEV)
    vc_d, dc_d = gu.to_dev(np.asarray(vc, np.float32)), gu.to_dev(np.asarray(dc, np.float32))
    B.dspark_survival(conf_d, surv, status)
    B.dspark_topb_select(surv, order, ss, rank)
    B.dspark_choose_budget(ss, n_sampling, T, num_reqs, vc_d, dc_d, b_star, best, obj, status)
    B.dspark_allocate(order, b_star, R, K, pl, off, vi, tokens=tok_d, ver_tokens=vt)
    torch.cuda.synchronize()
    return dict(surv=surv.cpu().numpy(), order=order.cpu().numpy(), sorted_surv=ss.cpu().numpy(),
                rank=rank.cpu().numpy().reshape(R, K), b_star=int(b_star.item()), best_obj=float(best.item()),
                obj=obj.cpu().numpy(), prefix_len=pl.cpu().numpy(), offsets=off.cpu().numpy(),
                ver_idx=vi.cpu().numpy(), ver_tokens=None if vt is None else vt.cpu().numpy(),
                status=int(status.item()))


def _check(conf, n_sampling, T, num_reqs, vc, dc, expect_status=0):
    R, K = conf.shape
    tokens = (np.arange(R * K, dtype=np.int32) * 7 % 50021).reshape(R, K)
    want = sched.schedule(conf, n_sampling, T, num_reqs, vc, dc, tokens=tokens)
    got = _stagewise(conf, n_sampling, T, num_reqs, vc, dc, tokens=tokens)
    gu.assert_sched_parity(got, want, R, K)
    np.testing.assert_array_equal(got["rank"], want["rank"])
    np.testing.assert_array_equal(got["obj"], want["obj"])
    assert got["status"] == want["status"] == expect_status
    return got


@pytest.mark.parametrize("name", ["tiny", "small", "mid", "headline", "large", "sweep"])
def test_workload_schedules_stagewise(name):
    w = inputs.WORKLOADS[name]
    gu.say(f"schedule {name} R={w.R} K={w.K} T={w.T}")
    conf = inputs._confidences(w, np.random.default_rng(w.seed * 7 + 1))
    rng = np.random.default_rng(w.seed)
    vc = sched.force_monotone(inputs.raw_verify_cost(w, rng))
    dc = sched.force_monotone(inputs.raw_draft_cost(w))
    got = _check(conf, w.n_sampling, w.T, w.R_all, vc, dc)
    assert 0 <= got["b_star"] <= w.R * w.K


def test_ties_zeros_and_ones():
    rng = np.random.default_rng(1)
    R, K = 700, 15
    conf = rng.choice(np.array([0.0, 0.25, 0.5, 0.75, 1.0], dtype=np.float32), size=(R, K))
    conf[::7] = 1.0            # whole rows of survival 1.0: many exact ties across requests
    conf[3::11, 0] = 0.0       # requests with nothing to verify
    vc = np.arange(16385, dtype=np.float32) * 0.05 + 1000.0
    dc = (300.0 + 2.0 * np.arange(1025)).astype(np.float32)
    _check(conf, R, 0, R, vc, dc)


def test_bad_confidences_are_sanitized_and_flagged():
    rng = np.random.default_rng(2)
    conf = rng.uniform(0, 1, size=(40, 7)).astype(np.float32)
    conf[0, 3] = np.nan
    conf[5, 0] = -0.5
    conf[7, 2] = 1.5
    conf[9, 1] = -0.0
    conf[11, :] = np.inf
    vc = (2000.0 + np.arange(600)).astype(np.float32)
    dc = (300.0 + 2.0 * np.arange(300)).astype(np.float32)
    _check(conf, 40, 3, 40, vc, dc, expect_status=B.STATUS_CONF_SANITIZED)


def test_no_room_for_drafts_and_no_sampling():
    rng = np.random.default_rng(3)
    conf = rng.uniform(0.3, 1, size=(12, 5)).astype(np.float32)
    vc = (100.0 + np.arange(20)).astype(np.float32)
    dc = (300.0 + 2.0 * np.arange(20)).astype(np.float32)
    got = _check(conf, 0, 19, 12, vc, dc)        # T = verify_len - 1: Bmax = 0
    assert got["b_star"] == 0 and got["best_obj"] == 0.0
    _check(conf, 0, 0, 12, vc, dc)               # n_sampling = 0


def test_invalid_costs_are_skipped_and_flagged():
    conf = np.full((6, 4), 0.8, dtype=np.float32)
    vc = np.full(40, 500.0, dtype=np.float32)
    vc[3] = np.nan
    vc[4] = -1.0
    vc[5] = np.inf
    dc = np.zeros(8, dtype=np.float32)
    _check(conf, 6, 0, 6, vc, dc, expect_status=B.STATUS_COST_INVALID)


@pytest.mark.parametrize("R,K", [(1, 1), (3, 1), (1, 15), (1023, 1), (65, 16), (16384, 1), (1024, 16)])
def test_shapes_up_to_the_slot_limit(R, K):
    w = inputs.WORKLOADS["large"]
    conf = inputs._confidences(inputs.Workload(**{**w.__dict__, "R": R, "K": K}), np.random.default_rng(R * K))
    vc = sched.force_monotone(inputs.raw_verify_cost(w, np.random.default_rng(4)))
    dc = np.maximum.accumulate((300.0 + 2.0 * np.arange(R + 1)).astype(np.float32))
    gu.say(f"schedule shape R={R} K={K}")
    _check(conf, R, 100, R, vc, dc)


def test_topb_matches_python_sorted_on_fresh_draws():
    for seed in range(3):
        rng = np.random.default_rng(50 + seed)
        surv = np.sort(rng.uniform(0, 1, size=(900, 13)).astype(np.float32), axis=1)[:, ::-1].copy()
        surv[rng.integers(0, 900, 50), :] = surv[0]   # duplicated rows
        R, K = surv.shape
        order = torch.empty(R * K, dtype=torch.int32, device=gu.DEV)
        ss = torch.empty(R * K, dtype=torch.float32, device=gu.DEV)
        B.dspark_topb_select(gu.to_dev(surv), order, ss)
        torch.cuda.synchronize()
        flat = surv.reshape(-1)
        want = sorted(range(R * K), key=lambda f: (-float(flat[f]), f))
        np.testing.assert_array_equal(order.cpu().numpy(), np.array(want, dtype=np.int32))


def _budget_gpu(ss, n_sampling, T, num_reqs, vc, dc, rule):
    n = len(ss)
    bmax = min(n, len(vc) - 1 - T)
    b_star = torch.empty(1, dtype=torch.int32, device=gu.DEV)
    best = torch.empty(1, dtype=torch.float64, device=gu.DEV)
    obj = torch.empty(bmax + 1, dtype=torch.float64, device=gu.DEV)
    status = torch.zeros(1, dtype=torch.int32, device=gu.DEV)
    ss_d = gu.to_dev(np.asarray(ss, np.float32)) if n else torch.empty(0, dtype=torch.float32, device=gu.DEV)
    B.dspark_choose_budget(ss_d, n_sampling, T, num_reqs, gu.to_dev(np.asarray(vc, np.float32)),
                           gu.to_dev(np.asarray(dc, np.float32)), b_star, best, obj, status, rule=rule)
    torch.cuda.synchronize()
    return int(b_star.item()), float(best.item()), obj.cpu().numpy(), int(status.item())


def _budget_cases():
    """(label, sorted survivals, n_sampling, T, num_reqs, vc, dc) over the shapes the rules differ on."""
    cases = []
    for name in ("tiny", "small", "mid", "headline", "large", "sweep"):
        w = inputs.WORKLOADS[name]
        for seed in range(2):
            rng = np.random.default_rng(300 + seed)
            conf = inputs._confidences(w, rng)
            ss = sched.topb_order(sched.survival(conf)[0])[1]
            vc = sched.force_monotone(inputs.raw_verify_cost(w, rng))
            dc = sched.force_monotone(inputs.raw_draft_cost(w))
            cases.append((f"{name}/{seed}", ss, w.n_sampling, w.T, w.R_all, vc, dc))
    rng = np.random.default_rng(8)
    for n, slope in ((16384, 0.02), (5000, 1.0), (1023, 3.0), (1, 0.5), (0, 1.0)):
        s = np.sort(rng.beta(3.0, 1.5, n).astype(np.float32))[::-1].copy()
        vc = (1000.0 + slope * np.arange(n + 40)).astype(np.float32)
        dc = np.full(8, 100.0, np.float32)
        cases.append((f"linear/{n}", s, 64, 3, 5, vc, dc))
    # plateaus: zero survivals under a flat cost; a staircase from the pages' cost model
    s = np.concatenate([np.full(700, 0.5, np.float32), np.zeros(600, np.float32)])
    cases.append(("plateau", s, 4, 0, 1, np.full(2000, 300.0, np.float32), np.full(4, 10.0, np.float32)))
    stair = np.array([2000.0 + 1.0 * inputs.pad_to_graph(t, 4096) for t in range(1500)], np.float32)
    cases.append(("stair", s, 4, 0, 1, stair, np.full(4, 10.0, np.float32)))
    # every B's cost is the same, so f only rises until the zeros: also no room at all
    cases.append(("no-room", s, 4, 1999, 1, np.full(2000, 300.0, np.float32), np.full(4, 10.0, np.float32)))
    return cases


@pytest.mark.parametrize("rule", [B.RULE_ARGMAX, B.RULE_FIRST_DROP])
def test_budget_rules_match_the_oracle(rule):
    differ = 0
    for label, ss, ns, T, nr, vc, dc in _budget_cases():
        gu.say(f"budget rule {rule}: {label} n={len(ss)}")
        b, best, obj, st = _budget_gpu(ss, ns, T, nr, vc, dc, rule)
        wb, wbest, wobj, wst = sched.choose_budget(ss, ns, T, nr, vc, dc, rule=rule)
        assert b == wb, (label, b, wb)
        assert best == wbest, (label, best, wbest)
        np.testing.assert_array_equal(obj, wobj)
        assert st == wst
        differ += wb != sched.choose_budget(ss, ns, T, nr, vc, dc)[0]
    if rule == B.RULE_FIRST_DROP:
        assert differ >= 3


@pytest.mark.parametrize("rule", [B.RULE_ARGMAX, B.RULE_FIRST_DROP])
@pytest.mark.parametrize("name", ["tiny", "small", "mid", "headline", "large", "sweep"])
def test_fused_schedule_entry_point(name, rule):
    # dspark_schedule: stages 2-5 in one kernel, on every workload's slots (the sweep is
    # 1024 requests x 15 positions), with verified tokens, then sized from another array.
    w = inputs.WORKLOADS[name]
    rng = np.random.default_rng(w.seed + 40)
    conf = inputs._confidences(w, rng)
    vc = sched.force_monotone(inputs.raw_verify_cost(w, np.random.default_rng(w.seed)))
    dc = sched.force_monotone(inputs.raw_draft_cost(w))
    R, K = conf.shape
    tokens = rng.integers(0, 50000, size=(R, K)).astype(np.int32)
    out = B.StepBuffers(R, K)
    status = torch.zeros(1, dtype=torch.int32, device=gu.DEV)
    args = (w.n_sampling, w.T, w.R_all, gu.to_dev(vc), gu.to_dev(dc), out)
    B.dspark_schedule(gu.to_dev(conf), *args, rule=rule, tokens=gu.to_dev(tokens), status=status)
    torch.cuda.synchronize()
    got = gu.step_numpy(out)
    want = sched.schedule(conf, w.n_sampling, w.T, w.R_all, vc, dc, tokens=tokens, rule=rule)
    gu.assert_sched_parity(got, want, R, K)
    assert int(status.item()) == want["status"] == 0
    old = inputs._confidences(w, np.random.default_rng(w.seed + 41))
    B.dspark_schedule(gu.to_dev(conf), *args, size_conf=gu.to_dev(old), rule=rule, status=status)
    torch.cuda.synchronize()
    got = gu.step_numpy(out)
    got["ver_tokens"] = None
    want = sched.schedule(conf, w.n_sampling, w.T, w.R_all, vc, dc, size_conf=old, rule=rule)
    gu.assert_sched_parity(got, want, R, K)
