#!/usr/bin/env python3
"""Benchmark of the chain-and-schedule step on one MI355X.

One step = the whole pass through dspark_step on one batch of synthetic inputs
already resident in HBM: the chain (stage 1), then stages 2-5 over the
confidences and the verified-token gather, in that order (the schedule starts
once the chain has ended, as in the method, where the confidences score the
drafted tokens).  Per-step inputs (base logits, prev0, confidences) cycle through
a pool of distinct seeded draws (far larger together than the 256 MB last-level
cache); the Markov-head factors and cost tables stay fixed, as weights and
start-up profiles do.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chain+schedule steps/sec at R=256,K=7,V=129280,r=256; % HBM roofline; sched µs"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0      # dense bf16 matrix cores
FP32_VECTOR_PEAK_TFLOPS = 157.3     # fp32 vector


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def step_bytes(w) -> dict:
    """Algorithmic HBM bytes of one step: every input read once, every output written once."""
    e = 2 if w.dtype == 1 else 4
    n = w.R * w.K
    bmax = min(n, w.verify_len - 1 - w.T)
    d = dict(base=w.R * w.K * w.V * e, factor_B=w.V * w.rank * e, factor_A_rows=n * w.rank * e,
             prev0=w.R * 4, conf=n * 4, cost=(bmax + 1) * 4 + 4,
             outputs=n * 4 * 6 + w.R * 4 + (w.R + 1) * 4 + 12)
    d["total"] = sum(d.values())
    return d


def chain_kernel(w, num_cu: int = 256, form: int = 0) -> dict:
    """The dominant kernel of the step and its algorithmic bytes per launch.  bf16 with
    K <= 32 and V <= 262144 in the pruned form (the default) runs stage 1 as one launch
    of cand_chain_kernel, whose algorithmic bytes are the chain's share of the step's:
    every base logit and the second factor once, the K*R key rows, prev0 and the tokens
    (the kernel itself reads the base logits and only the candidates' factor rows).
    Otherwise: bf16 with
    R <= 256, and fp32 with R <= 64 and rank <= 64, run the whole step in one launch of a
    resident grid (step_single_bf16_kernel, step_single_f32_kernel): every base logit
    once, the second factor once, the K*R gathered key rows, the keys written and read
    back, the confidences, cost-table entries and every output once.  Otherwise one chain
    launch per position moves its base slice, the whole second factor, its R key rows and
    keys."""
    e = 2 if w.dtype == 1 else 4
    if form == 0 and w.dtype == 1 and w.K <= 32 and w.V <= 262144:
        b = w.R * w.K * w.V * e + w.V * w.rank * e + w.R * w.K * w.rank * e + w.R * 4 + w.R * w.K * 4
        return {"kernel": "cand_chain_kernel", "bytes_per_launch": b, "launches_per_step": 1}
    tiles = (w.V + 511) // 512  # one 512-entry vocabulary tile per workgroup, one workgroup per CU
    single = (w.R <= 256) if w.dtype == 1 else (w.R <= 64 and w.rank <= 64)
    if single and tiles + 1 <= num_cu:
        b = step_bytes(w)["total"] + w.R * w.K * 8 * 2
        name = "step_single_bf16_kernel" if w.dtype == 1 else "step_single_f32_kernel"
        return {"kernel": name, "bytes_per_launch": b, "launches_per_step": 1}
    if w.dtype == 1 and (w.R <= 256 and tiles <= num_cu or w.R <= 64 and tiles <= 2 * num_cu):
        # the whole chain in one launch (two vocabulary tiles per workgroup past num_cu
        # tiles); the schedule runs in its own launch.  Algorithmic bytes: base, both
        # factors' used rows and the keys once, though the two-tile form reads half of the
        # second factor again at every position after the first.
        b = (w.R * w.K * w.V * e + w.V * w.rank * e + w.R * w.K * w.rank * e + w.R * 4 + w.R * w.K * (8 * 2 + 4))
        name = "chain_persist_bf16_kernel" if tiles <= num_cu else "chain_persist2_bf16_kernel"
        return {"kernel": name, "bytes_per_launch": b, "launches_per_step": 1}
    b = w.R * w.V * e + w.V * w.rank * e + w.R * w.rank * e + w.R * (8 * 2 + 4)
    name = "chain_pos_bf16_kernel" if w.dtype == 1 else "chain_pos_f32_kernel"
    return {"kernel": name, "bytes_per_launch": b, "launches_per_step": w.K}


def traffic_per_launch(kernel: str, workload: str):
    """Measured HBM bytes per launch of `kernel` at `workload` from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by its plain-copy calibration), or None
    when the counters were taken at another workload or any source of the kernel has
    changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or not rec.get("workload", "").startswith(workload + ":"):
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(round(rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]))


def host_info() -> dict:
    """The host the oracle is timed on: its logical CPU count and model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cpus": os.cpu_count(), "host_cpu_model": model}


def cpu_baseline(w, ins, step_in, vc, dc, rows: int) -> dict:
    """The oracle as it stands, timed on this host: the chain of `rows` requests (all
    positions, whole vocabulary) scaled to R requests, plus the full schedule."""
    import oracle
    from oracle import sched
    # one core, enforced: the oracle is single-threaded and is timed as such
    cores = None
    try:
        before = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(before)})
        cores = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        before = None
    sel = np.linspace(0, w.R - 1, rows).astype(np.int32)
    t0 = time.perf_counter()
    oracle.chain(step_in["base"], ins.A, ins.Bmat, w.dtype, step_in["prev0"], rows=sel)
    t_chain = time.perf_counter() - t0
    t0 = time.perf_counter()
    sched.schedule(step_in["conf"], w.n_sampling, w.T, w.R_all, vc, dc)
    t_sched = time.perf_counter() - t0
    per_step = t_chain * (w.R / rows) + t_sched
    if before is not None:
        os.sched_setaffinity(0, before)
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": cores or 1, "kind": "oracle",
            "affinity": "pinned to one core (sched_setaffinity)" if cores else "not pinned", **host_info(),
            "sample": f"fp64 chain of {rows} of {w.R} requests (all {w.K} positions, V={w.V}) timed "
                      f"{t_chain:.2f} s and scaled x{w.R / rows:.0f}; schedule of all {w.R * w.K} slots "
                      f"timed {t_sched:.2f} s; single-threaded"}


def copy_bandwidth(dev, mib: int = 1024, reps: int = 10) -> float:
    """Read + write GB/s of a plain device-to-device copy: the practical streaming peak."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def _event_loop_us(fn, n: int) -> float:
    """Mean microseconds per call of fn(k), k < n, from one event pair around the loop."""
    import torch
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(n):
        fn(k)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def accept_lane(w, B, inputs, out, st, dev, calls: int = 200) -> dict:
    """The greedy acceptance lane on the last step's allocation, with a synthetic target
    whose acceptance is drawn from that step's confidences; timed and checked."""
    import torch
    from oracle import verify
    ver = out.ver_tokens.cpu().numpy()
    offsets = out.offsets.cpu().numpy()
    target = inputs.synthetic_target(ver, offsets, st["conf"], w.V, seed=12345)
    tgt = torch.from_numpy(target).to(dev)
    i32 = dict(dtype=torch.int32, device=dev)
    a, p, o = torch.empty(w.R, **i32), torch.empty(w.R, **i32), torch.empty((w.R, w.K + 1), **i32)
    stat = torch.zeros(1, **i32)

    def run(_k):
        B.dspark_accept_greedy(out.ver_tokens, out.offsets, tgt, w.R, w.K, a, p, o, stat)

    for k in range(5):
        run(k)
    us = _event_loop_us(run, calls)
    wa, wp, wo, _ = verify.accept_greedy(ver, offsets, target, w.R, w.K)
    ok = (np.array_equal(a.cpu().numpy(), wa) and np.array_equal(p.cpu().numpy(), wp)
          and np.array_equal(o.cpu().numpy(), wo) and int(stat.item()) == 0)
    log(f"bench: acceptance lane {us:.2f} us/call, parity {'ok' if ok else 'MISMATCH'}")
    return {"us_per_call": round(us, 2), "calls": calls, "accepted_per_step": int(wa.sum()),
            "emitted_per_step": int(wa.sum()) + w.R, "verified_per_step": int(offsets[-1]),
            "parity": "ok" if ok else "MISMATCH"}


def stale_sized(w, B, osched, pool, host_steps, mk, vc_d, dc_d, vc, dc, out, ws, status, rule, steps) -> dict:
    """dspark_step_sized with B sized from the previous pool entry's confidences (a
    one-step-old buffer) under `rule`; timed over `steps` steps and checked on the last."""
    P = len(pool)
    plan = B.StepPlan(mk, w.R, w.K, w.n_sampling, w.T, w.R_all, vc_d, dc_d, out, ws, status, rule=rule)

    def run(k):
        base, prev0, conf = pool[k % P]
        plan(base, prev0, conf, pool[(k - 1) % P][2])

    for k in range(10):
        run(k)
    us = _event_loop_us(run, steps)
    k = steps - 1
    want = osched.schedule(host_steps[k % P]["conf"], w.n_sampling, w.T, w.R_all, vc, dc,
                           size_conf=host_steps[(k - 1) % P]["conf"], rule=rule)
    same = osched.schedule(host_steps[k % P]["conf"], w.n_sampling, w.T, w.R_all, vc, dc, rule=rule)
    ok = (int(out.b_star.item()) == want["b_star"] and float(out.best_obj.item()) == want["best_obj"]
          and np.array_equal(out.ver_idx.cpu().numpy(), want["ver_idx"]))
    log(f"bench: stale sizing rule {rule}: {us:.1f} us/step, B {want['b_star']} (same-step {same['b_star']}), "
        f"parity {'ok' if ok else 'MISMATCH'}")
    return {"step_us": round(us, 2), "steps_per_s": round(1e6 / us, 1), "steps": steps,
            "b_last": int(want["b_star"]), "b_same_step": int(same["b_star"]), "parity": "ok" if ok else "MISMATCH"}


def sampled_chain(w, B, pool, host_steps, ins, mk, ws, dev, steps) -> dict:
    """Stage 1 with probabilistic drafting (dspark_chain_sample, temperature 1.0, a new
    seed every step): one launch per position of the general scorer with a Gumbel
    variate (Philox4x32-10 + two logarithms) per vocabulary entry; timed, and one row of
    the last step checked against the oracle's sampled chain."""
    import torch
    import oracle
    P = len(pool)
    tokens = torch.empty((w.R, w.K), dtype=torch.int32, device=dev)

    def run(k):
        base, prev0, _ = pool[k % P]
        B.dspark_chain_sample(base, mk, prev0, 1.0, 1000 + k, tokens, None, None, ws)

    for k in range(3):
        run(k)
    us = _event_loop_us(run, steps)
    k = steps - 1
    st = host_steps[k % P]
    tok = tokens.cpu().numpy()
    otok, pert, _ = oracle.chain_sample(st["base"], ins.A, ins.Bmat, w.dtype, st["prev0"], 1.0, 1000 + k, rows=[0],
                                        forced=tok, want_perturbed=True)
    ok = True
    for i in range(w.K):
        if otok[0, i] != tok[0, i]:
            yo, yg = pert[0, i, otok[0, i]], pert[0, i, tok[0, i]]
            ok &= bool(yo - yg <= 1e-4 * max(abs(yo), 1.0))
    elems = w.R * w.K * w.V
    log(f"bench: sampled chain {us:.1f} us/step ({elems / us / 1e3:.1f} G entries/s), parity {'ok' if ok else 'MISMATCH'}")
    return {"step_us": round(us, 2), "steps": steps, "temperature": 1.0,
            "entries_per_s": round(elems / (us * 1e-6), 1), "philox_calls_per_step": elems // 4,
            "parity_row0": "ok" if ok else "MISMATCH"}


def sched_kernel_us(B, pool, w, vc_d, dc_d, dev, calls) -> float:
    """Stages 2-5 alone through dspark_schedule (one 1024-thread workgroup) on the pool's
    confidences; mean microseconds per call.  The step itself runs them over many
    workgroups when its slots allow (a ranking launch, then a one-workgroup finish), and
    event_pass.after_chain_us times that part of the step."""
    import torch
    out = B.StepBuffers(w.R, w.K, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    P = len(pool)

    def run(k):
        B.dspark_schedule(pool[k % P][-1], w.n_sampling, w.T, w.R_all, vc_d, dc_d, out, status=st)

    for k in range(5):
        run(k)
    us = _event_loop_us(run, calls)
    log(f"bench: schedule kernel alone {us:.1f} us per call")
    return round(us, 2)


def sched_only(args, w, B, inputs, osched, dev):
    """Scheduler-only workload (no chain): one step = dspark_schedule over all R*K slots."""
    import torch
    log(f"bench: scheduler-only workload {w.name} R={w.R} K={w.K} ({w.R * w.K} slots)")
    ins = inputs.generate(w)
    vc = B.dspark_force_monotone(ins.verify_cost_raw)
    dc = B.dspark_force_monotone(ins.draft_cost_raw)
    vc_d, dc_d = torch.from_numpy(vc).to(dev), torch.from_numpy(dc).to(dev)
    host = [inputs.generate_step(w, k) for k in range(args.pool)]
    pool = [(torch.from_numpy(h["conf"]).to(dev),) for h in host]
    out = B.StepBuffers(w.R, w.K, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(k):
        B.dspark_schedule(pool[k % len(pool)][0], w.n_sampling, w.T, w.R_all, vc_d, dc_d, out, status=status)

    for k in range(args.warmup):
        run(k)
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        run(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = _event_loop_us(run, min(args.event_steps, K))
    # the last call of the event loop wrote `out`
    want = osched.schedule(host[(min(args.event_steps, K) - 1) % len(pool)]["conf"], w.n_sampling, w.T, w.R_all,
                           vc, dc)
    ok = (int(out.b_star.item()) == want["b_star"] and float(out.best_obj.item()) == want["best_obj"]
          and np.array_equal(out.ver_idx.cpu().numpy(), want["ver_idx"])
          and np.array_equal(out.order.cpu().numpy(), want["order"]))
    n = w.R * w.K
    bmax = min(n, w.verify_len - 1 - w.T)
    nbytes = n * 4 + (bmax + 1) * 4 + 4 + n * 4 * 4 + w.R * 4 + (w.R + 1) * 4 + 12
    ach = nbytes / (us * 1e-6) / 1e9
    res = {"metric": "schedule steps/sec (stages 2-5 alone)", "value": round(K / wall, 2), "unit": "steps/s",
           "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / K, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{w.name}: R={w.R}, K={w.K} ({n} slots), T={w.T}, N_sampling={w.n_sampling}"},
           "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 6), "traffic": None, "kernel": "sched_fused_kernel",
                        "bytes_per_launch": nbytes, "launch_us": round(us, 2),
                        "note": "one workgroup out of LDS; bound by its sort and scan latency, not by HBM"},
           "sched_kernel_us": round(us, 2), "parity_last_step": "ok" if ok else "MISMATCH",
           "status": int(status.item())}
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        osched.schedule(host[0]["conf"], w.n_sampling, w.T, w.R_all, vc, dc)
        t = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": 1.0 / t, "unit": "steps/s", "cores": 1, "kind": "oracle", **host_info(),
                               "sample": f"the whole schedule of {n} slots, timed {t:.2f} s; single-threaded"}
    print(json.dumps(res), flush=True)


def dense_forms(B, run, steps) -> dict:
    """The same step in the dense form (the matrix-core chain over the whole vocabulary,
    with stages 2-5 on a workgroup of the same single launch, beside the chain), launched
    as a plain launch of a resident grid and cooperatively."""
    out = {}
    B.dspark_set_chain_form(B.CHAIN_DENSE)
    try:
        for label, mode in (("dense_overlapped", B.LAUNCH_RESIDENT), ("dense_overlapped_cooperative",
                                                                      B.LAUNCH_COOPERATIVE)):
            B.dspark_set_launch_mode(mode)
            for k in range(10):
                run(k)
            us = _event_loop_us(run, steps)
            log(f"bench: {label} {us:.1f} us/step")
            out[label] = {"step_us": round(us, 2), "steps_per_s": round(1e6 / us, 1), "steps": steps}
    finally:
        B.dspark_set_launch_mode(B.LAUNCH_RESIDENT)
        B.dspark_set_chain_form(B.CHAIN_PRUNED)
    return out


def vocab_shard(B, inputs, dev, steps) -> dict:
    """One GPU's share of the headline chain under an 8-way vocabulary split (V / 8 =
    16160 columns, all 256 requests): the step's chain and schedule on that shard, pruned
    and dense.  (Across GPUs each position's keys would meet in one small max all-reduce,
    which one GPU does not show.)"""
    import torch
    w = inputs.WORKLOADS["shard"]
    ins = inputs.generate(w)

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    mk = B.MarkovHead(d(ins.A), d(ins.Bmat), w.dtype)
    vc_d = d(B.dspark_force_monotone(ins.verify_cost_raw))
    dc_d = d(B.dspark_force_monotone(ins.draft_cost_raw))
    base, prev0, conf = d(ins.base), d(ins.prev0), d(ins.conf)
    ws = B.workspace(w.R, w.K, w.V, w.rank, w.dtype, device=dev)
    out = B.StepBuffers(w.R, w.K, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    plan = B.StepPlan(mk, w.R, w.K, w.n_sampling, w.T, w.R_all, vc_d, dc_d, out, ws, st)
    res = {"workload": f"{w.name}: R={w.R}, K={w.K}, V={w.V}, r={w.rank}"}
    for label, form in (("pruned", B.CHAIN_PRUNED), ("dense", B.CHAIN_DENSE)):
        B.dspark_set_chain_form(form)
        try:
            for _ in range(10):
                plan(base, prev0, conf)
            us = _event_loop_us(lambda k: plan(base, prev0, conf), steps)
        finally:
            B.dspark_set_chain_form(B.CHAIN_PRUNED)
        res[label] = {"step_us": round(us, 2), "steps_per_s": round(1e6 / us, 1)}
        log(f"bench: vocabulary shard ({label}) {us:.1f} us/step")
    res["status"] = int(st.item())
    return res


def closed_loop(w, B, pool, mk, vc_d, dc_d, ws, dev, steps) -> dict:
    """A multi-step synthetic decode loop, all on the device: each iteration runs the step
    sized from the previous step's confidences (dspark_step_sized), a stand-in for the
    target model's greedy tokens whose acceptance is drawn from this step's confidences
    (torch ops: draft j of a request matches with probability c[r, j], the bonus token is
    uniform), the acceptance lane (dspark_accept_greedy), and keys the next step's chain on
    the bonus tokens.  Reports the emitted tokens (accepted drafts + one bonus per request)."""
    import torch
    R, K, V, n = w.R, w.K, w.V, w.R * w.K
    P = len(pool)
    out = B.StepBuffers(R, K, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    prev0 = pool[0][1].clone()
    acc_len, nxt = torch.empty(R, **i32), torch.empty(R, **i32)
    target = torch.zeros(n + R + 1, **i32)       # the last entry takes the writes of unused slots
    emitted = torch.zeros(1, dtype=torch.int64, device=dev)
    j = torch.arange(n, device=dev)
    rr = torch.arange(R, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2026)

    def one(k):
        base, _, conf = pool[k % P]
        old = pool[(k - 1) % P][2]
        B.dspark_step_sized(base, mk, prev0, conf, old, B.RULE_ARGMAX, w.n_sampling, w.T, w.R_all, vc_d, dc_d,
                            out, ws, status)
        slot = out.ver_idx.long()
        valid = j < out.b_star.long()
        slot_c = slot.clamp(min=0)
        req = slot_c // K
        c = conf.reshape(-1)[slot_c]
        u = torch.rand(n, device=dev, generator=gen)
        other = torch.randint(1, V, (n,), device=dev, generator=gen, dtype=torch.int32)
        draft = out.ver_tokens
        answer = torch.where(u < c, draft, torch.remainder(draft + other, V))
        dst = torch.where(valid, j + req, torch.full_like(j, n + R))
        target.index_copy_(0, dst, answer)
        bonus = torch.randint(0, V, (R,), device=dev, generator=gen, dtype=torch.int32)
        target.index_copy_(0, out.offsets[1:].long() + rr, bonus)
        B.dspark_accept_greedy(out.ver_tokens, out.offsets, target, R, K, acc_len, nxt, None, status)
        emitted.add_(acc_len.sum() + R)
        prev0.copy_(nxt)

    for k in range(5):
        one(k)
    emitted.zero_()
    us = _event_loop_us(one, steps)
    per_step = float(emitted.item()) / steps
    log(f"bench: closed loop {us:.1f} us/iteration, {per_step:.1f} emitted tokens per step "
        f"({per_step / (us * 1e-6) / 1e6:.2f} M tokens/s), status {int(status.item())}")
    return {"iteration_us": round(us, 2), "steps": steps, "emitted_tokens_per_step": round(per_step, 1),
            "emitted_tokens_per_s": round(per_step / (us * 1e-6), 1), "status": int(status.item()),
            "sizing": "one-step-old confidences, argmax rule",
            "target": "synthetic stand-in (torch): draft j accepted with probability c[r, j]"}


def measured_tables(w, B, osched, pool, host_steps, mk, out, ws, status, dev) -> dict:
    """Cost tables measured on this GPU at start-up: a proxy verification step (4 bf16
    GEMMs [t, 7168] x [7168, 7168]) over the captured sizes up to the workload's capture
    limit plus 1.5x and 2x above it, and a proxy drafting step (one GEMM over the K
    draft tokens of each request) by request count; median of 5 runs each; then one step
    sized with them, checked against the oracle on the same tables."""
    import torch
    from confidence_scheduled_verification_amd import costmodel
    t0 = time.perf_counter()
    vproxy = costmodel.GemmProxy(max_tokens=2 * w.graph_max, hidden=7168, layers=4, device=dev)
    vc, vshapes, vs = costmodel.measure_table(vproxy, w.graph_max, w.verify_len)
    del vproxy
    dproxy = costmodel.GemmProxy(max_tokens=2 * (w.draft_len - 1) * w.K, hidden=7168, layers=1, device=dev, seed=1)
    dc, dshapes, ds = costmodel.measure_table(lambda n: dproxy(n * w.K), w.draft_len - 1, w.draft_len)
    del dproxy
    torch.cuda.empty_cache()
    build_s = time.perf_counter() - t0
    base, prev0, conf = pool[0]
    vc_d, dc_d = torch.from_numpy(vc).to(dev), torch.from_numpy(dc).to(dev)
    B.dspark_step(base, mk, prev0, conf, w.n_sampling, w.T, w.R_all, vc_d, dc_d, out, ws, status)
    torch.cuda.synchronize()
    want = osched.schedule(host_steps[0]["conf"], w.n_sampling, w.T, w.R_all, vc, dc)
    ok = (int(out.b_star.item()) == want["b_star"] and float(out.best_obj.item()) == want["best_obj"]
          and np.array_equal(out.ver_idx.cpu().numpy(), want["ver_idx"]))
    log(f"bench: measured tables in {build_s:.1f} s; B = {want['b_star']} with them, parity {'ok' if ok else 'MISMATCH'}")
    med = lambda x: [round(float(np.median(r)), 1) for r in x]
    return {"verify_shapes": vshapes, "verify_median_us": med(vs), "draft_shapes": dshapes,
            "draft_median_us": med(ds), "proxy": "4 x bf16 GEMM [t,7168]x[7168,7168] (verify); 1 x GEMM over "
            f"{w.K} tokens per request (draft)", "build_s": round(build_s, 2), "b_star": int(want["b_star"]),
            "best_obj": want["best_obj"], "parity": "ok" if ok else "MISMATCH"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="headline", choices=["tiny", "small", "mid", "headline", "large", "shard", "sweep"])
    ap.add_argument("--pool", type=int, default=4, help="distinct per-step input sets cycled through")
    ap.add_argument("--cpu-rows", type=int, default=128, help="requests in the oracle's timed chain sample")
    ap.add_argument("--event-steps", type=int, default=200,
                    help="steps of the second pass that times the kernels with HIP events")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the timed variants (stale sizing, sampling, acceptance, measured tables)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times): under rocprofv3 --pmc its "
                         "FETCH_SIZE / WRITE_SIZE per dispatch calibrate the HBM traffic counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the chain-and-schedule step has "
                                   "no multi-GPU path (it would shard by requests, which are independent, "
                                   "or by vocabulary, with one 64-bit max all-reduce of the keys per position)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    from confidence_scheduled_verification_amd import binding as B
    from confidence_scheduled_verification_amd import inputs
    from oracle import sched as osched

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(3)
    B.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": n, "dispatches": 5}), flush=True)
        return
    w = inputs.WORKLOADS[args.workload]
    if not w.has_chain:
        return sched_only(args, w, B, inputs, osched, dev)
    log(f"bench: workload {w.name} R={w.R} K={w.K} V={w.V} rank={w.rank}; generating inputs")
    ins = inputs.generate(w)
    vc = B.dspark_force_monotone(ins.verify_cost_raw)
    dc = B.dspark_force_monotone(ins.draft_cost_raw)

    def dev_t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    mk = B.MarkovHead(dev_t(ins.A), dev_t(ins.Bmat), w.dtype)
    vc_d, dc_d = dev_t(vc), dev_t(dc)
    pool, host_steps = [], []
    for k in range(args.pool):
        st = inputs.generate_step(w, k)
        host_steps.append(st)
        pool.append((dev_t(st["base"]), dev_t(st["prev0"]), dev_t(st["conf"])))
        log(f"bench: pool entry {k} uploaded")
    ws = B.workspace(w.R, w.K, w.V, w.rank, w.dtype, device=dev)
    out = B.StepBuffers(w.R, w.K, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    # every argument that stays fixed across steps is marshalled once: a step is one C call
    plan = B.StepPlan(mk, w.R, w.K, w.n_sampling, w.T, w.R_all, vc_d, dc_d, out, ws, status)

    def run(k):
        base, prev0, conf = pool[k % len(pool)]
        plan(base, prev0, conf)

    for k in range(args.warmup):
        run(k)
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done; timing {args.steps}")

    # Pass 1 (the reported value): K steps between synchronizations, wall clock and one
    # event pair around the whole loop (per-step events would add their own cost).
    K = args.steps
    stream = torch.cuda.current_stream()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for k in range(K):
        run(k)
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    loop_ms = g0.elapsed_time(g1)
    log(f"bench: wall {wall * 1e3 / K:.2f} ms/step, events {loop_ms * 1e3 / K:.1f} us/step")

    # Pass 2: the same steps with HIP events set by the library around the chain on the
    # step's stream, for the kernel-level roofline (for the pruned chain they take the
    # kernel's own start and stop time; otherwise they are markers around its launches).
    KE = max(1, min(args.event_steps, K))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(KE)]
    for e in ev:
        # torch creates the HIP event on its first record; the library re-records
        # e[1] and e[2] inside each step (dspark_set_timing_events)
        e[1].record(stream)
        e[2].record(stream)
    torch.cuda.synchronize()
    for k in range(KE):
        e0, e1, e2, e3 = ev[k]
        e0.record(stream)
        B.dspark_set_timing_events(e1, e2)
        run(k)
        e3.record(stream)
    torch.cuda.synchronize()
    B.dspark_set_timing_events(None, None)
    step_ms = np.array([ev[k][0].elapsed_time(ev[k][3]) for k in range(KE)])
    pre_ms = np.array([ev[k][0].elapsed_time(ev[k][1]) for k in range(KE)])
    chain_ms = np.array([ev[k][1].elapsed_time(ev[k][2]) for k in range(KE)])
    post_ms = np.array([ev[k][2].elapsed_time(ev[k][3]) for k in range(KE)])
    log(f"bench: event pass {KE} steps: {step_ms.mean() * 1e3:.1f} us/step "
        f"(chain {chain_ms.mean() * 1e3:.1f} us, after it {post_ms.mean() * 1e3:.1f} us)")

    # Parity against the oracle (every chain row + the whole schedule) on steps 0, 1, 499
    # and the last of the timed sequence, each run again untimed (a step's result
    # depends only on its inputs, which cycle through the pool).
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    def rows_ok(st, tok, rows) -> bool:
        # teacher-forced oracle on these rows; a differing token must be an oracle near-tie
        otok, _, _ = oracle.chain(st["base"], ins.A, ins.Bmat, w.dtype, st["prev0"], rows=rows, forced=tok)
        bad = [q for q in range(len(rows)) if not np.array_equal(otok[q], tok[rows[q]])]
        if not bad:
            return True
        sel = np.asarray(rows)[bad]
        otok, olog, _ = oracle.chain(st["base"], ins.A, ins.Bmat, w.dtype, st["prev0"], rows=sel, forced=tok,
                                     want_logits=True)
        ok = True
        for q, r in enumerate(sel):
            for i in range(w.K):
                if otok[q, i] != tok[r, i]:
                    xo, xg = olog[q, i, otok[q, i]], olog[q, i, tok[r, i]]
                    ok &= bool(xo - xg <= 1e-4 * max(abs(xo), 1.0))
        return ok

    def check(k) -> bool:
        # every chain row (threads: the C oracle releases the interpreter lock) and the schedule
        st = host_steps[k % len(pool)]
        tok = out.tokens.cpu().numpy()
        nthr = max(1, min(16, os.cpu_count() or 1))
        chunks = np.array_split(np.arange(w.R, dtype=np.int32), min(w.R, 4 * nthr))
        with ThreadPoolExecutor(max_workers=nthr) as ex:
            ok = all(ex.map(lambda rows: rows_ok(st, tok, rows), [c for c in chunks if len(c)]))
        want = osched.schedule(st["conf"], w.n_sampling, w.T, w.R_all, vc, dc)
        ok &= int(out.b_star.item()) == want["b_star"]
        ok &= float(out.best_obj.item()) == want["best_obj"]
        ok &= np.array_equal(out.ver_idx.cpu().numpy(), want["ver_idx"])
        ok &= np.array_equal(out.order.cpu().numpy(), want["order"])
        return ok

    checked = {}
    for k in sorted({k for k in (0, 1, 499, K - 1) if 0 <= k < K}):
        run(k)
        torch.cuda.synchronize()
        checked[k] = check(k)
    ok = all(checked.values())
    parity = "ok" if ok else "MISMATCH"
    log(f"bench: parity of steps {sorted(checked)}: {parity}")

    sched_us = sched_kernel_us(B, pool, w, vc_d, dc_d, dev, min(args.event_steps, K))
    extra = None
    if not args.no_variants:
        extra = {"accept_greedy": accept_lane(w, B, inputs, out, st, dev)}
        extra.update(dense_forms(B, run, min(args.event_steps, K)))
        for label, rule in (("stale_sizing_argmax", B.RULE_ARGMAX), ("stale_sizing_first_drop", B.RULE_FIRST_DROP)):
            extra[label] = stale_sized(w, B, osched, pool, host_steps, mk, vc_d, dc_d, vc, dc, out, ws, status,
                                       rule, min(args.event_steps, K))
        extra["sampled_chain"] = sampled_chain(w, B, pool, host_steps, ins, mk, ws, dev,
                                               min(args.event_steps, 100))
        extra["measured_cost_tables"] = measured_tables(w, B, osched, pool, host_steps, mk, out, ws, status, dev)
        extra["closed_loop"] = closed_loop(w, B, pool, mk, vc_d, dc_d, ws, dev, min(args.event_steps, K))
        if w.name == "headline":
            extra["vocab_shard"] = vocab_shard(B, inputs, dev, min(args.event_steps, K))

    copy_gbs = copy_bandwidth(dev)
    log(f"bench: plain device copy {copy_gbs:.0f} GB/s (read + write)")
    sb = step_bytes(w)
    ck = chain_kernel(w, torch.cuda.get_device_properties(0).multi_processor_count, B.dspark_get_chain_form())
    launch_s = chain_ms.mean() * 1e-3 / ck["launches_per_step"]   # event-timed chain phase per launch
    achieved = ck["bytes_per_launch"] / launch_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_per_launch(ck["kernel"], w.name), **ck,
                "launch_us": round(launch_s * 1e6, 2),
                "practical_peak": {"kind": "plain device copy, 1 GiB read + 1 GiB written", "gbs": round(copy_gbs, 1),
                                   "frac": round(achieved / copy_gbs, 4)}}
    # the dense contraction's flop count over the chain's time; the pruned form evaluates
    # the bias for the candidates alone, so this is the work it avoids, not work it does
    flops = 2.0 * w.R * w.K * w.V * w.rank
    pruned = ck["kernel"] == "cand_chain_kernel"
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == 1 else FP32_VECTOR_PEAK_TFLOPS
    mfma_tf = flops / (chain_ms.mean() * 1e-3) / 1e12
    compute = {"unit": "TFLOP/s", "flops_per_step": flops, "achieved": round(mfma_tf, 1), "peak": mfma_peak,
               "frac": round(mfma_tf / mfma_peak, 4),
               "engine": ("none: the bias is evaluated for the candidates only (fp32 FMA); this is the dense "
                          "contraction's flop count per chain time" if pruned else
                          ("bf16 MFMA" if w.dtype == 1 else "fp32 vector FMA"))}
    ms_per_step = wall * 1e3 / K
    res = {
        "metric": METRIC,
        "value": round(K / wall, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: R={w.R} (of {w.R_all}), K={w.K}, V={w.V}, r={w.rank}, T={w.T}, "
                               f"N_sampling={w.n_sampling}", "input_pool": len(pool),
                   "order": ("serial: the chain, then stages 2-5 over the confidences (two launches, one stream)"
                             if pruned else "one launch: stages 2-5 on a workgroup beside the chain"),
                   "chain_form": "pruned" if pruned else "dense"},
        "roofline": roofline,
        "compute": compute,
        "sched_kernel_us": sched_us,
        "step_bytes": sb["total"],
        "step_hbm_frac": round(sb["total"] / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "step_us_loop_events": round(loop_ms * 1e3 / K, 2),
        # the step in the method's order: the chain, then stages 2-5 over the confidences
        # (the reported value is this serial step; no part of the schedule overlaps the chain)
        "serial_step_us": round(ms_per_step * 1e3, 2) if pruned else None,
        "event_pass": {"steps": KE, "step_us": round(float(step_ms.mean()) * 1e3, 2),
                       "before_chain_us": round(float(pre_ms.mean()) * 1e3, 2),
                       "chain_us": round(float(chain_ms.mean()) * 1e3, 2),
                       "after_chain_us": round(float(post_ms.mean()) * 1e3, 2),
                       "note": ("chain_us: the pruned chain kernel's own start to stop (its launch carries "
                                "the events), else markers around the chain launches; the markers before "
                                "and after the step add their own time to the other parts")},
        "parity_last_step": "ok" if checked[K - 1] else "MISMATCH",
        "parity": parity,
        "parity_steps": {str(k): ("ok" if v else "MISMATCH") for k, v in sorted(checked.items())},
        "status": int(status.item()),
        "variants": extra,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(w, ins, host_steps[0], vc, dc, min(args.cpu_rows, w.R))
    print(json.dumps(res), flush=True)
    # Orderly teardown before the interpreter exits: no library-held event handles, every
    # queued kernel done, device buffers released while the runtime is fully up.
    B.dspark_set_timing_events(None, None)
    torch.cuda.synchronize()
    del plan, pool, out, ws, status, mk, ev
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
