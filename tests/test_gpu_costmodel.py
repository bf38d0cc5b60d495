"""Cost tables measured on this GPU: the library times a proxy step (bf16 GEMMs) over the
captured sizes plus sizes above them, builds the forced staircase tables, and the budget
chosen from them on the GPU matches the oracle's on the same tables bit for bit."""
import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import costmodel, inputs
from oracle import costs, sched

pytestmark = pytest.mark.gpu


def test_measured_tables_feed_the_budget():
    gu.say("profiling a GEMM proxy over graph sizes 1..512 and 768, 1024")
    proxy = costmodel.GemmProxy(max_tokens=1024, hidden=2048, layers=2)
    vc, shapes, samples = costmodel.measure_table(proxy, graph_max=512, table_len=1025)
    assert shapes == [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 768, 1024]
    assert samples.shape == (len(shapes), 5) and np.all(samples > 0) and np.all(np.isfinite(samples))
    np.testing.assert_array_equal(vc, costs.build_cost_table(shapes, samples, 512, 1025))
    assert np.all(np.diff(vc) >= 0)
    for lo, hi in zip(shapes[:-3], shapes[1:-2]):          # staircase between captured sizes
        assert np.all(vc[lo + 1:hi + 1] == vc[hi])
    gu.say("profiling the drafter proxy by request count")
    K = 7
    dproxy = costmodel.GemmProxy(max_tokens=64 * K * 2, hidden=1024, layers=1, seed=1)
    dc, dshapes, _ = costmodel.measure_table(lambda n: dproxy(n * K), graph_max=64, table_len=65, above=(2.0,))
    assert dshapes[-1] == 128 and np.all(np.diff(dc) >= 0)
    R = 64
    conf = inputs._confidences(inputs.WORKLOADS["small"], np.random.default_rng(2))
    conf = np.concatenate([conf, conf])[:R].copy()
    ss = sched.topb_order(sched.survival(conf)[0])[1]
    b_star = torch.empty(1, dtype=torch.int32, device=gu.DEV)
    best = torch.empty(1, dtype=torch.float64, device=gu.DEV)
    for rule in (B.RULE_ARGMAX, B.RULE_FIRST_DROP):
        B.dspark_choose_budget(gu.to_dev(ss), R, 0, R, gu.to_dev(vc), gu.to_dev(dc), b_star, best, rule=rule)
        torch.cuda.synchronize()
        wb, wf, _, _ = sched.choose_budget(ss, R, 0, R, vc, dc, rule=rule)
        assert int(b_star.item()) == wb and float(best.item()) == wf, rule
        gu.say(f"rule {rule}: B = {wb} of {R * K} slots on the measured tables")


def test_a_failing_proxy_step_is_reported():
    def step(t):
        if t > 4:
            raise RuntimeError("proxy failed")
    with pytest.raises(RuntimeError, match="proxy failed"):
        B.dspark_profile_shapes(step, [1, 2, 4, 8], runs=2, warmup=0)
