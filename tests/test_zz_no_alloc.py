"""dspark_step_static (the step for callers that cannot allocate: its workspace is a
static array in the library) against dspark_step with a caller's workspace, on the same
inputs: every output bit for bit, on two calls in a row, the second with a smaller
batch; fp32 factors and both chain forms (the dense forms keep counters and keys in the
workspace, the pruned chain keeps nothing there)."""
import dataclasses

import numpy as np
import pytest
import torch

import gpu_util as gu
from confidence_scheduled_verification_amd import binding as B
from confidence_scheduled_verification_amd import inputs

pytestmark = pytest.mark.gpu

FIELDS = ["tokens", "surv", "order", "sorted_surv", "b_star", "best_obj", "prefix_len", "offsets", "ver_idx",
          "ver_tokens"]


def _step(w, ins, ch, static):
    vc, dc = gu.forced_tables(w, ins)
    conf = gu.to_dev(np.asarray(ins.conf, dtype=np.float32))
    vc_d, dc_d = gu.to_dev(np.asarray(vc, dtype=np.float32)), gu.to_dev(np.asarray(dc, dtype=np.float32))
    out = B.StepBuffers(w.R, w.K)
    for f in FIELDS:
        getattr(out, f).fill_(-7)  # a result left unwritten shows as a mismatch
    status = torch.zeros(1, dtype=torch.int32, device=gu.DEV)
    if static:
        B.dspark_step_static(ch.base, ch.markov, ch.prev0, conf, w.n_sampling, w.T, w.R_all, vc_d, dc_d, out,
                             status)
    else:
        B.dspark_step(ch.base, ch.markov, ch.prev0, conf, w.n_sampling, w.T, w.R_all, vc_d, dc_d, out, ch.ws,
                      status)
    torch.cuda.synchronize()
    return {f: getattr(out, f).cpu().numpy().copy() for f in FIELDS}, int(status.item())


@pytest.mark.parametrize("name,form,rows", [("tiny", "dense", (4, 3)), ("small", "dense", (32, 19)),
                                            ("small", "pruned", (32, 19))])
def test_static_workspace_step_equals_the_workspace_step(name, form, rows):
    with gu.chain_form(gu.FORMS[form]):
        for R in rows:  # two calls in a row on the same static array, the second smaller
            w = dataclasses.replace(inputs.WORKLOADS[name], R=R, R_all=R)
            gu.say(f"step_static {name} {form}: R={R} K={w.K} V={w.V}")
            ins = inputs.generate(w)
            ch = gu.Chain(ins.base, ins.A, ins.Bmat, w.dtype, ins.prev0)
            want, s_want = _step(w, ins, ch, static=False)
            got, s_got = _step(w, ins, ch, static=True)
            assert s_want == 0 and s_got == 0
            for f in FIELDS:
                np.testing.assert_array_equal(got[f], want[f], err_msg=f"{name} {form} R={R}: {f}")
