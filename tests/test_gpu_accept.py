"""GPU parity of the greedy acceptance lane (dspark_accept_greedy) against the oracle,
on its own over ragged layouts and in a closed multi-step loop: step, a synthetic
target whose acceptance is drawn from the confidences, acceptance, and the next
step keyed on the bonus tokens.  Every comparison is bit-exact."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import inputs
from oracle import sched, verify

pytestmark = pytest.mark.gpu


def _accept_gpu(ver, offsets, target, R, K, with_tokens=True):
    i32 = dict(dtype=torch.int32, device=gu.DEV)
    a = torch.full((R,), -7, **i32)
    prev = torch.full((R,), -7, **i32)
    out = torch.full((R, K + 1), -7, **i32) if with_tokens else None
    status = torch.zeros(1, **i32)
    B.dspark_accept_greedy(gu.to_dev(np.asarray(ver, np.int32)), gu.to_dev(np.asarray(offsets, np.int32)),
                           gu.to_dev(np.asarray(target, np.int32)), R, K, a, prev, out, status)
    torch.cuda.synchronize()
    return (a.cpu().numpy(), prev.cpu().numpy(), None if out is None else out.cpu().numpy(),
            int(status.item()))


def _planted(seed, R, K, V=1000, bad_rows=()):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, K + 1, size=R)
    L[rng.random(R) < 0.2] = K
    offsets = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    ver = np.full(R * K, -1, np.int32)
    ver[:offsets[-1]] = rng.integers(0, V, size=offsets[-1])
    target = rng.integers(0, V, size=R * K + R).astype(np.int32)
    for r in range(R):
        o, n = offsets[r], L[r]
        cut = rng.integers(0, n + 1)
        target[o + r:o + r + cut] = ver[o:o + cut]
        if cut < n:
            target[o + r + cut] = (ver[o + cut] + 1) % V
    for r in bad_rows:
        offsets[r + 1] = offsets[r] - 1 if r % 2 else offsets[r] + K + 1
    return ver, offsets, target


@pytest.mark.parametrize("R,K", [(1, 1), (4, 7), (257, 7), (300, 3), (64, 15), (33, 64), (20, 100), (9, 130),
                                 (1000, 1), (5, 0)])
def test_accept_matches_the_oracle(R, K):
    gu.say(f"accept R={R} K={K}")
    ver, offsets, target = _planted(R * 1000 + K, R, K)
    a, prev, out, st = _accept_gpu(ver, offsets, target, R, K)
    wa, wp, wo, wst = verify.accept_greedy(ver, offsets, target, R, K)
    np.testing.assert_array_equal(a, wa)
    np.testing.assert_array_equal(prev, wp)
    np.testing.assert_array_equal(out, wo)
    assert st == wst == 0
    a2, prev2, none, _ = _accept_gpu(ver, offsets, target, R, K, with_tokens=False)
    assert none is None and np.array_equal(a2, wa) and np.array_equal(prev2, wp)


def test_inconsistent_rows_are_flagged():
    R, K = 40, 7
    ver, offsets, target = _planted(5, R, K, bad_rows=(3, 10))
    a, prev, out, st = _accept_gpu(ver, offsets, target, R, K)
    wa, wp, wo, wst = verify.accept_greedy(ver, offsets, target, R, K)
    assert wst == st == B.STATUS_BAD_ALLOCATION
    np.testing.assert_array_equal(a, wa)
    np.testing.assert_array_equal(prev, wp)
    np.testing.assert_array_equal(out, wo)


@pytest.mark.parametrize("name,steps", [("small", 4), ("headline", 2)])
def test_closed_loop_of_steps(name, steps):
    # step k's bonus tokens key step k+1's chain; acceptance is drawn from step k's confidences
    w = inputs.WORKLOADS[name]
    ins = inputs.generate(w)
    vc, dc = gu.forced_tables(w, ins)
    ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
    out = B.StepBuffers(w.R, w.K)
    prev0 = ins.prev0.copy()
    i32 = dict(dtype=torch.int32, device=gu.DEV)
    a_d, p_d = torch.empty(w.R, **i32), torch.empty(w.R, **i32)
    emitted = 0
    for k in range(steps):
        gu.say(f"loop {name} step {k}")
        st = inputs.generate_step(w, k)
        ch.base.copy_(gu.to_dev(st["base"]))
        ch.prev0.copy_(gu.to_dev(prev0))
        got, status, _ = gu.run_step(ch, st["conf"], w.n_sampling, w.T, w.R_all, vc, dc, out=out)
        assert status == 0
        gu.assert_chain_parity(got["tokens"], None, st["base"], ins.A, ins.Bmat, w.dtype, prev0)
        want = sched.schedule(st["conf"], w.n_sampling, w.T, w.R_all, vc, dc, tokens=got["tokens"])
        gu.assert_sched_parity(got, want, w.R, w.K)
        target = inputs.synthetic_target(got["ver_tokens"], got["offsets"], st["conf"], w.V, seed=500 + k)
        status_d = torch.zeros(1, **i32)
        B.dspark_accept_greedy(out.ver_tokens, out.offsets, gu.to_dev(target), w.R, w.K, a_d, p_d, None, status_d)
        torch.cuda.synchronize()
        wa, wp, _, wst = verify.accept_greedy(want["ver_tokens"], want["offsets"], target, w.R, w.K)
        np.testing.assert_array_equal(a_d.cpu().numpy(), wa)
        np.testing.assert_array_equal(p_d.cpu().numpy(), wp)
        assert int(status_d.item()) == wst == 0
        assert np.all((wp >= 0) & (wp < w.V))
        emitted += int(wa.sum()) + w.R
        prev0 = p_d.cpu().numpy()
    assert emitted > steps * w.R
