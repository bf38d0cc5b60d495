"""ORACLE -- test infrastructure only (tests, smoke check and the CPU-baseline leg).

Greedy verification of the allocated drafts, written out plainly.

Under greedy decoding a draft token is accepted exactly when it equals the
target model's best token at that position (MAX worklog "DSpark on MAX", section
"The kernel pass", item 2), and the verifier keeps the longest run of leading
drafts that match (DSpark summary "How DSpark Speeds Up LLM Inference", section
"Context").  Every request also gains one token from the target itself -- the
bonus token of the budget's numerator (vLLM blog "Adaptive Verification in
vLLM", section "Scheduling the budget") -- which is the target's token right
after the accepted run, and which the next step's chain is keyed on.

Layout readings:
  * request r's verified drafts are ver_tokens[offsets[r] .. offsets[r+1]), the
    compacted list of the allocation stage, L_r = offsets[r+1] - offsets[r];
  * the target pass runs 1 + L_r tokens per request (the last accepted token and
    the L_r drafts; vLLM blog, section "Varlen decode CUDA graphs": each request
    may carry between 1 and k+1 tokens), so its greedy tokens for request r are
    target[offsets[r] + r .. offsets[r] + r + L_r], entry j being the target's
    choice after the request's first j drafts;
  * accepted a_r = the number of leading j < L_r with draft j == target entry j;
    the bonus token is target entry a_r; the emitted tokens are the a_r accepted
    drafts followed by the bonus token; the next step's prev0 is the bonus token;
  * an allocation row that is inconsistent (negative offset or length, length
    above K, past R*K) accepts nothing, emits nothing, gets prev0 = -1 and sets
    status bit 16.
"""
from __future__ import annotations

import numpy as np

STATUS_BAD_ALLOCATION = 16


def accept_greedy(ver_tokens, offsets, target, R, K):
    """Returns (accept_len [R], next_prev0 [R], out_tokens [R, K+1] padded with -1, status)."""
    ver_tokens = np.asarray(ver_tokens, dtype=np.int64).reshape(-1)
    offsets = np.asarray(offsets, dtype=np.int64).reshape(-1)
    target = np.asarray(target, dtype=np.int64).reshape(-1)
    accept_len = np.zeros(R, dtype=np.int32)
    next_prev0 = np.full(R, -1, dtype=np.int32)
    out_tokens = np.full((R, K + 1), -1, dtype=np.int32)
    status = 0
    for r in range(R):
        o = int(offsets[r])
        L = int(offsets[r + 1]) - o
        if o < 0 or L < 0 or L > K or o + L > R * K:
            status |= STATUS_BAD_ALLOCATION
            continue
        drafts = [int(ver_tokens[o + j]) for j in range(L)]
        answers = [int(target[o + r + j]) for j in range(L + 1)]
        a = 0
        while a < L and drafts[a] == answers[a]:
            a += 1
        accept_len[r] = a
        next_prev0[r] = answers[a]
        for j in range(a):
            out_tokens[r, j] = drafts[j]
        out_tokens[r, a] = answers[a]
    return accept_len, next_prev0, out_tokens, status
