"""ORACLE -- test infrastructure only (tests, smoke check and the CPU-baseline leg).

Stages 2-5 of the chain-and-schedule step and the start-up cost-table forcing,
written out in the order the vLLM blog "Adaptive Verification in vLLM" gives
them (section "Scheduling the budget"; section "The cost model" for the tables).
Plain Python loops over plain numbers: float32 products through numpy scalars,
sums of survivals as exact rationals (``fractions.Fraction``), IEEE double
division through Python floats.

Readings of what the pages leave open:
  * survival is the inclusive running product s[r,i] = c[r,0] * ... * c[r,i]
    (the confidence is the chance a token survives given that all before it
    were accepted -- DSpark summary, "Verify smarter" -- so s[r,i] is the chance
    that the first i+1 drafts all survive), in float32, in increasing i;
  * a confidence that is NaN or below 0 becomes 0, one above 1 becomes 1, and
    status bit 2 is set; -0.0 becomes +0.0 silently;
  * slots are ranked by survival descending, then request ascending, then
    position ascending;
  * B runs over 0 .. min(R*K, verify_len - 1 - T); the objective is
    f(B) = fl64(N_sampling + S_B) / fl64(vc[T+B] + dc[num_reqs]) where S_B is
    the exact sum of the B best survivals (rounded once to double together with
    N_sampling) and the division is IEEE double; the smallest B among equal
    maxima wins (np.argmax returns the first maximum);
  * a cost sum that is not a positive finite number makes that B's objective
    -inf and sets status bit 4;
  * the compacted verification list holds flat slot ids r*K+i, ordered by
    request then position, padded with -1 to R*K entries;
  * the first-drop admission rule (AlphaSignal's DSpark summary "How DSpark
    Speeds Up LLM Inference", section "Verify smarter": slots enter in rank
    order for as long as each one raises the throughput, and the first one that
    would lower it ends admission) admits slot B+1 only when f(B+1) > f(B) strictly, so it stops at
    the smallest B of a plateau, as the argmax rule does;
  * stale sizing (vLLM blog, "Scheduling the budget": B is sized from a
    confidence array one step old while the slots are handed out with current
    values; the DSpark summary's production notes speak of two steps): B is
    chosen from the older array's survivals with the current step's scalars and
    cost tables, then capped at the current slot count, and the current ranking's
    first B slots are allocated.  best_obj is the sizing objective f(B) before
    the cap.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

STATUS_PREV_CLAMPED = 1
STATUS_CONF_SANITIZED = 2
STATUS_COST_INVALID = 4

RULE_ARGMAX = 0       # B* = smallest B maximising f (vLLM blog, "Scheduling the budget")
RULE_FIRST_DROP = 1   # admit while f rises (DSpark summary, "Verify smarter")


def force_monotone(table):
    """Start-up forcing of a profiled cost table: each entry becomes the running maximum
    of the entries up to it (vLLM blog, "The cost model": profiling noise is removed by
    forcing the curve monotonic).  Entries must be finite."""
    out = [float(np.float32(x)) for x in table]
    for x in out:
        if not math.isfinite(x):
            raise ValueError("cost table entries must be finite")
    for t in range(1, len(out)):
        if out[t] < out[t - 1]:
            out[t] = out[t - 1]
    return np.array(out, dtype=np.float32)


def _sanitize(c):
    c = np.float32(c)
    if math.isnan(float(c)) or float(c) < 0.0:
        return np.float32(0.0), True
    if float(c) > 1.0:
        return np.float32(1.0), True
    if float(c) == 0.0:
        return np.float32(0.0), False      # -0.0 -> +0.0
    return c, False


def survival(conf):
    """Stage 2: s[r,0] = c[r,0]; s[r,i] = fl32(s[r,i-1] * c[r,i]).  Returns (surv, status)."""
    conf = np.asarray(conf, dtype=np.float32)
    R, K = conf.shape
    surv = np.zeros((R, K), dtype=np.float32)
    status = 0
    for r in range(R):
        s = None
        for i in range(K):
            c, bad = _sanitize(conf[r, i])
            if bad:
                status |= STATUS_CONF_SANITIZED
            s = c if i == 0 else np.float32(s * c)
            surv[r, i] = s
    return surv, status


def topb_order(surv):
    """Stage 3: all R*K slots ranked by (survival desc, request asc, position asc).

    Returns (order [n] flat ids r*K+i, sorted_surv [n] float32, rank [R,K])."""
    surv = np.asarray(surv, dtype=np.float32)
    R, K = surv.shape
    flat = [float(x) for x in surv.reshape(-1)]
    order = sorted(range(R * K), key=lambda f: (-flat[f], f))
    order = np.array(order, dtype=np.int32)
    sorted_surv = surv.reshape(-1)[order] if R * K else np.zeros(0, dtype=np.float32)
    rank = np.zeros(R * K, dtype=np.int32)
    rank[order] = np.arange(R * K, dtype=np.int32)
    return order, sorted_surv.astype(np.float32), rank.reshape(R, K)


def choose_budget(sorted_surv, n_sampling, T, num_reqs, verify_cost, draft_cost, rule=RULE_ARGMAX):
    """Stage 4: the budget B in [0, Bmax].

    RULE_ARGMAX: the smallest B maximising f(B) (vLLM blog, "Scheduling the budget").
    RULE_FIRST_DROP: starting from B = 0, slots are admitted one at a time in rank
    order while the objective strictly rises; B is where the next admission would
    not raise it, or Bmax (DSpark summary "How DSpark Speeds Up LLM Inference",
    section "Verify smarter").

    Returns (b, f(b), obj [Bmax+1] float64, status)."""
    if rule not in (RULE_ARGMAX, RULE_FIRST_DROP):
        raise ValueError("unknown admission rule")
    n = len(sorted_surv)
    verify_len = len(verify_cost)
    if not (0 <= T < verify_len) or not (0 <= num_reqs < len(draft_cost)) or n_sampling < 0:
        raise ValueError("scheduler scalars out of range")
    bmax = min(n, verify_len - 1 - T)
    dc = float(np.float32(draft_cost[num_reqs]))
    obj = np.zeros(bmax + 1, dtype=np.float64)
    status = 0
    S = Fraction(0)
    for B in range(bmax + 1):
        if B > 0:
            S += Fraction(float(sorted_surv[B - 1]))      # S is now the sum of the B best
        num = float(Fraction(n_sampling) + S)
        den = float(np.float32(verify_cost[T + B])) + dc
        if math.isfinite(den) and den > 0.0:
            f = num / den
        else:
            f = -math.inf
            status |= STATUS_COST_INVALID
        obj[B] = f
    if rule == RULE_ARGMAX:
        best_b = 0
        for B in range(1, bmax + 1):
            if obj[B] > obj[best_b]:
                best_b = B
    else:
        best_b = 0
        while best_b < bmax and obj[best_b + 1] > obj[best_b]:
            best_b += 1
    return best_b, float(obj[best_b]), obj, status


def allocate(order, b_star, R, K, tokens=None):
    """Stage 5: the B* best slots handed to their requests.

    Returns (prefix_len [R], offsets [R+1], ver_idx [R*K], ver_tokens [R*K] or None).
    prefix_len[r] counts request r's selected slots; offsets is their exclusive
    running sum; ver_idx lists the selected flat ids by request then position and
    is padded with -1; ver_tokens[j] = tokens.flat[ver_idx[j]] (or -1)."""
    n = R * K
    selected = [False] * n
    for j in range(b_star):
        selected[int(order[j])] = True
    prefix_len = np.zeros(R, dtype=np.int32)
    for r in range(R):
        prefix_len[r] = sum(1 for i in range(K) if selected[r * K + i])
    offsets = np.zeros(R + 1, dtype=np.int32)
    for r in range(R):
        offsets[r + 1] = offsets[r] + prefix_len[r]
    ver_idx = np.full(n, -1, dtype=np.int32)
    j = 0
    for f in range(n):
        if selected[f]:
            ver_idx[j] = f
            j += 1
    ver_tokens = None
    if tokens is not None:
        flat_tok = np.asarray(tokens, dtype=np.int32).reshape(-1)
        ver_tokens = np.full(n, -1, dtype=np.int32)
        for j in range(b_star):
            ver_tokens[j] = flat_tok[ver_idx[j]]
    return prefix_len, offsets, ver_idx, ver_tokens


def schedule(conf, n_sampling, T, num_reqs, verify_cost, draft_cost, tokens=None, size_conf=None,
             rule=RULE_ARGMAX):
    """Stages 2-5 in order.  Returns a dict of every intermediate and output.

    size_conf (optional, [R', K]): the confidences B is sized from, e.g. those of one
    or two steps earlier; the current conf is then used for the ranking and the
    allocation only, and B is capped at R*K (vLLM blog, "Scheduling the budget")."""
    conf = np.asarray(conf, dtype=np.float32)
    R, K = conf.shape
    surv, st2 = survival(conf)
    order, sorted_surv, rank = topb_order(surv)
    st_size = 0
    if size_conf is None:
        b_star, best_obj, obj, st4 = choose_budget(sorted_surv, n_sampling, T, num_reqs, verify_cost, draft_cost,
                                                   rule)
    else:
        size_conf = np.asarray(size_conf, dtype=np.float32).reshape(-1, K)
        size_surv, st_size = survival(size_conf)
        _, size_sorted, _ = topb_order(size_surv)
        b_size, best_obj, obj, st4 = choose_budget(size_sorted, n_sampling, T, num_reqs, verify_cost, draft_cost,
                                                   rule)
        b_star = min(b_size, R * K)
    prefix_len, offsets, ver_idx, ver_tokens = allocate(order, b_star, R, K, tokens)
    return dict(surv=surv, order=order, sorted_surv=sorted_surv, rank=rank, b_star=b_star,
                best_obj=best_obj, obj=obj, prefix_len=prefix_len, offsets=offsets, ver_idx=ver_idx,
                ver_tokens=ver_tokens, status=st2 | st4 | st_size)
