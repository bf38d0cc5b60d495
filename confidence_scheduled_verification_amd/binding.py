"""Thin Python binding of libdspark.so (include/dspark.h).

Argument marshalling only: every function here checks shapes, takes device
pointers from torch tensors and calls the C entry point of the same name on the
current (or given) HIP stream.  No step of the method runs in Python.  The
library is loaded on first use and a missing library raises immediately -- there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdspark.so")

DSPARK_F32 = 0
DSPARK_BF16 = 1
STATUS_PREV_CLAMPED = 1
STATUS_CONF_SANITIZED = 2
STATUS_COST_INVALID = 4
STATUS_SYNC_TIMEOUT = 8
STATUS_BAD_ALLOCATION = 16
LAUNCH_RESIDENT = 0
LAUNCH_COOPERATIVE = 1
MAX_SLOTS = 16384
RULE_ARGMAX = 0
RULE_FIRST_DROP = 1
CHAIN_PRUNED = 0
CHAIN_DENSE = 1
MARKOV_MAGIC = 0x31766b6d6b707364
MARKOV_HEADER_BYTES = 256

EXPORTS = ["dspark_last_error", "dspark_version", "dspark_workspace_bytes", "dspark_markov_state_bytes",
           "dspark_markov_prepare", "dspark_set_chain_form", "dspark_get_chain_form",
           "dspark_chain", "dspark_chain_sample", "dspark_survival", "dspark_topb_select", "dspark_choose_budget", "dspark_allocate",
           "dspark_step", "dspark_step_sized", "dspark_step_static", "dspark_schedule", "dspark_accept_greedy", "dspark_set_timing_events",
           "dspark_force_monotone", "dspark_profile_shapes", "dspark_build_cost_table", "dspark_set_launch_mode",
           "dspark_get_launch_mode"]

# int fn(int shape, void* user, void* stream)
SHAPE_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p)


class dspark_markov_t(ctypes.Structure):
    """The C handle of a prepared Markov head (include/dspark.h)."""
    _fields_ = [("magic", ctypes.c_uint64), ("A", ctypes.c_void_p), ("Bmat", ctypes.c_void_p),
                ("state", ctypes.c_void_p), ("state_bytes", ctypes.c_size_t), ("V", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class DSparkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libdspark error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libdspark.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m "
                               "confidence_scheduled_verification_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.dspark_last_error.restype = ctypes.c_char_p
        L.dspark_last_error.argtypes = []
        L.dspark_version.restype = ctypes.c_char_p
        L.dspark_version.argtypes = []
        L.dspark_workspace_bytes.restype = sz
        L.dspark_workspace_bytes.argtypes = [i, i, i, i, i]
        L.dspark_markov_state_bytes.restype = sz
        L.dspark_markov_state_bytes.argtypes = [i, i, i]
        L.dspark_markov_prepare.argtypes = [p, p, p, i, i, i, p, sz, p]
        L.dspark_set_chain_form.argtypes = [i]
        L.dspark_get_chain_form.argtypes = []
        L.dspark_chain.argtypes = [p, p, p, i, p, i, i, i, i, p, p, p, p, p, sz, p]
        L.dspark_chain_sample.argtypes = [p, p, p, i, p, i, i, i, i, p, ctypes.c_float, ctypes.c_uint64, p, p, p,
                                          p, sz, p]
        L.dspark_survival.argtypes = [p, i, i, p, p, p]
        L.dspark_topb_select.argtypes = [p, i, i, p, p, p, p]
        L.dspark_choose_budget.argtypes = [p, i, i, i, i, p, i, p, i, i, p, p, p, p, p]
        L.dspark_allocate.argtypes = [p, p, i, i, p, p, p, p, p, p]
        L.dspark_step.argtypes = [p, p, p, i, p, i, i, i, i, p, p, i, i, i, p, i, p, i, p, p, p, p, p, p, p, p,
                                  p, p, p, p, sz, p]
        L.dspark_step_static.argtypes = [p, p, p, i, p, i, i, i, i, p, p, i, i, i, p, i, p, i, p, p, p, p, p, p,
                                         p, p, p, p, p, p]
        L.dspark_step_sized.argtypes = [p, p, p, i, p, i, i, i, i, p, p, p, i, i, i, i, i, p, i, p, i, p, p, p,
                                        p, p, p, p, p, p, p, p, p, sz, p]
        L.dspark_accept_greedy.argtypes = [p, p, p, i, i, p, p, p, p, p]
        L.dspark_schedule.argtypes = [p, i, i, p, i, i, i, i, i, p, i, p, i, p, p, p, p, p, p, p, p, p, p, p, p]
        L.dspark_set_timing_events.argtypes = [p, p]
        L.dspark_set_launch_mode.argtypes = [i]
        L.dspark_get_launch_mode.argtypes = []
        L.dspark_force_monotone.argtypes = [p, i]
        L.dspark_profile_shapes.argtypes = [SHAPE_FN, p, p, i, i, i, p, p]
        L.dspark_build_cost_table.argtypes = [p, i, p, i, i, p, i]
        for name in EXPORTS:
            if name not in ("dspark_last_error", "dspark_version", "dspark_workspace_bytes",
                            "dspark_markov_state_bytes"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise DSparkError(rc, lib().dspark_last_error().decode())


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("libdspark takes densely packed (contiguous) tensors")


def _elem_ok(t, dtype: int, what: str):
    want = 2 if dtype == DSPARK_BF16 else 4
    if t.element_size() != want:
        raise ValueError(f"{what}: expected {want}-byte elements for dtype {dtype}")


def dspark_version() -> str:
    return lib().dspark_version().decode()


def dspark_workspace_bytes(R: int, K: int, V: int, rank: int, dtype: int) -> int:
    return int(lib().dspark_workspace_bytes(R, K, V, rank, dtype))


class MarkovHead:
    """The Markov head's factors A [V, rank] and Bmat [rank, V] (device tensors, kept
    referenced here) with the library's prepared state (the transposed factor and the
    bias bound, in a device buffer owned here) and the handle the chain and step calls
    take (dspark_markov_prepare)."""

    def __init__(self, A, Bmat, dtype: int, stream=None):
        import torch
        if A.dim() != 2 or Bmat.dim() != 2:
            raise ValueError("MarkovHead: A must be [V, rank] and Bmat [rank, V]")
        V, rank = A.shape
        if tuple(Bmat.shape) != (rank, V):
            raise ValueError(f"MarkovHead: Bmat must be [rank, V] = [{rank}, {V}], got {tuple(Bmat.shape)}")
        _contig(A, Bmat)
        _elem_ok(A, dtype, "A")
        _elem_ok(Bmat, dtype, "Bmat")
        nbytes = int(lib().dspark_markov_state_bytes(V, rank, dtype))
        self.state = torch.empty(nbytes + 256, dtype=torch.uint8, device=A.device)
        pad = (-self.state.data_ptr()) % 256  # the library wants 256-byte alignment
        self._state_ptr = self.state.data_ptr() + pad
        self.A, self.Bmat, self.dtype, self.V, self.rank = A, Bmat, dtype, V, rank
        self.handle = dspark_markov_t()
        _check(lib().dspark_markov_prepare(ctypes.byref(self.handle), _p(A), _p(Bmat), V, rank, dtype,
                                           self._state_ptr, nbytes, _stream(stream)))
        self._ref = ctypes.byref(self.handle)

    @property
    def Bt(self):
        """The prepared transposed factor [V, rank] (a view into the state)."""
        import torch
        off = self._state_ptr - self.state.data_ptr() + MARKOV_HEADER_BYTES
        esz = 2 if self.dtype == DSPARK_BF16 else 4
        raw = self.state[off:off + self.V * self.rank * esz]
        return raw.view(torch.int16 if esz == 2 else torch.float32).view(self.V, self.rank)


def dspark_markov_prepare(A, Bmat, dtype: int, stream=None) -> MarkovHead:
    """Start-up preparation of the Markov head (see MarkovHead)."""
    return MarkovHead(A, Bmat, dtype, stream)


def dspark_set_chain_form(form: int):
    """Stage 1's form for later calls: CHAIN_PRUNED (default) or CHAIN_DENSE."""
    _check(lib().dspark_set_chain_form(form))


def dspark_get_chain_form() -> int:
    return int(lib().dspark_get_chain_form())


def _shape(t, want, what):
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{what} must be {list(want)}, got {list(t.shape)}")


def _chain_checks(base, markov: MarkovHead, prev0, tokens, chained_logits, what):
    if base.dim() != 3:
        raise ValueError(f"{what}: base must be [R, K, V]")
    R, K, V = base.shape
    if V != markov.V:
        raise ValueError(f"{what}: base has V={V}, the Markov head V={markov.V}")
    _shape(prev0, (R,), f"{what}: prev0")
    _shape(tokens, (R, K), f"{what}: tokens")
    if chained_logits is not None:
        _shape(chained_logits, (R, K, V), f"{what}: chained_logits")
    _contig(base, prev0, tokens, chained_logits)
    _elem_ok(base, markov.dtype, "base")
    if prev0.element_size() != 4 or tokens.element_size() != 4:
        raise ValueError(f"{what}: prev0 and tokens must be int32")
    return R, K, V


def _ws_bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def dspark_chain(base, markov: MarkovHead, prev0, tokens, chained_logits=None, status=None, ws=None, stream=None):
    R, K, V = _chain_checks(base, markov, prev0, tokens, chained_logits, "dspark_chain")
    _check(lib().dspark_chain(_p(base), _p(markov.A), _p(markov.Bmat), markov.dtype, _p(prev0), R, K, V,
                              markov.rank, markov._ref, _p(tokens), _p(chained_logits), _p(status), _p(ws),
                              _ws_bytes(ws), _stream(stream)))


def dspark_chain_sample(base, markov: MarkovHead, prev0, temperature: float, seed: int, tokens, chained_logits=None,
                        status=None, ws=None, stream=None):
    """Stage 1 with Gumbel-max sampling of softmax(x / temperature) (Philox4x32-10 keyed on seed)."""
    R, K, V = _chain_checks(base, markov, prev0, tokens, chained_logits, "dspark_chain_sample")
    _check(lib().dspark_chain_sample(_p(base), _p(markov.A), _p(markov.Bmat), markov.dtype, _p(prev0), R, K, V,
                                     markov.rank, markov._ref, float(temperature),
                                     int(seed) & 0xFFFFFFFFFFFFFFFF, _p(tokens), _p(chained_logits), _p(status),
                                     _p(ws), _ws_bytes(ws), _stream(stream)))


def dspark_survival(conf, surv, status=None, stream=None):
    R, K = conf.shape
    if tuple(surv.shape) != (R, K):
        raise ValueError("dspark_survival: surv must match conf")
    _contig(conf, surv)
    _check(lib().dspark_survival(_p(conf), R, K, _p(surv), _p(status), _stream(stream)))


def dspark_topb_select(surv, order, sorted_surv, rank=None, stream=None):
    R, K = surv.shape
    _contig(surv, order, sorted_surv, rank)
    if order.numel() != R * K or sorted_surv.numel() != R * K or (rank is not None and rank.numel() != R * K):
        raise ValueError("dspark_topb_select: outputs need R*K entries")
    _check(lib().dspark_topb_select(_p(surv), R, K, _p(order), _p(sorted_surv), _p(rank), _stream(stream)))


def dspark_choose_budget(sorted_surv, n_sampling: int, T: int, num_reqs: int, verify_cost, draft_cost, b_star,
                         best_obj, obj=None, status=None, stream=None, rule: int = RULE_ARGMAX):
    n = sorted_surv.numel()
    _contig(sorted_surv, verify_cost, draft_cost, obj)
    _check(lib().dspark_choose_budget(_p(sorted_surv), n, n_sampling, T, num_reqs, _p(verify_cost),
                                      verify_cost.numel(), _p(draft_cost), draft_cost.numel(), rule, _p(b_star),
                                      _p(best_obj), _p(obj), _p(status), _stream(stream)))


def dspark_allocate(order, b_star, R: int, K: int, prefix_len, offsets, ver_idx, tokens=None, ver_tokens=None,
                    stream=None):
    _contig(order, prefix_len, offsets, ver_idx, tokens, ver_tokens)
    if order.numel() != R * K or prefix_len.numel() != R or offsets.numel() != R + 1 or ver_idx.numel() != R * K:
        raise ValueError("dspark_allocate: inconsistent sizes")
    _check(lib().dspark_allocate(_p(order), _p(b_star), R, K, _p(tokens), _p(prefix_len), _p(offsets),
                                 _p(ver_idx), _p(ver_tokens), _stream(stream)))


def _step_checks(base, markov: MarkovHead, prev0, conf, verify_cost, draft_cost, out: "StepBuffers", ws, status,
                 what, need_ws=True):
    R, K, V = _chain_checks(base, markov, prev0, out.tokens, None, what)
    _shape(conf, (R, K), f"{what}: conf")
    for t, n in ((conf, "conf"), (verify_cost, "verify_cost"), (draft_cost, "draft_cost")):
        if t.dtype != _torch().float32:
            raise ValueError(f"{what}: {n} must be float32")
    _contig(conf, verify_cost, draft_cost)
    n = R * K
    for t, want, name in ((out.order, n, "order"), (out.ver_idx, n, "ver_idx"), (out.ver_tokens, n, "ver_tokens"),
                          (out.surv, n, "surv"), (out.sorted_surv, n, "sorted_surv"), (out.prefix_len, R, "prefix_len"),
                          (out.offsets, R + 1, "offsets"), (out.b_star, 1, "b_star"), (out.best_obj, 1, "best_obj")):
        if t.numel() < want:
            raise ValueError(f"{what}: out.{name} holds {t.numel()} entries, {want} needed")
    if status is not None and (status.numel() < 1 or status.element_size() != 4):
        raise ValueError(f"{what}: status must hold one 32-bit word")
    # (the library checks the workspace's size: dspark_workspace_bytes is what it can use
    # best, and a smaller one down to the shape's minimum is accepted)
    if need_ws and ws is None:
        raise ValueError(f"{what}: a workspace is needed")
    return R, K, V


def _torch():
    import torch
    return torch


def dspark_step(base, markov: MarkovHead, prev0, conf, n_sampling: int, T: int, num_reqs: int, verify_cost,
                draft_cost, out: "StepBuffers", ws, status=None, stream=None):
    """The whole pass (chain + schedule) into the buffers of `out`."""
    R, K, V = _step_checks(base, markov, prev0, conf, verify_cost, draft_cost, out, ws, status, "dspark_step")
    _check(lib().dspark_step(_p(base), _p(markov.A), _p(markov.Bmat), markov.dtype, _p(prev0), R, K, V, markov.rank,
                             markov._ref, _p(conf), n_sampling, T, num_reqs, _p(verify_cost), verify_cost.numel(),
                             _p(draft_cost), draft_cost.numel(), _p(out.tokens), _p(out.surv), _p(out.order),
                             _p(out.sorted_surv), _p(out.b_star), _p(out.best_obj), _p(out.prefix_len),
                             _p(out.offsets), _p(out.ver_idx), _p(out.ver_tokens), _p(status), _p(ws),
                             _ws_bytes(ws), _stream(stream)))


def dspark_step_static(base, markov: MarkovHead, prev0, conf, n_sampling: int, T: int, num_reqs: int, verify_cost,
                       draft_cost, out: "StepBuffers", status=None, stream=None):
    """dspark_step with the library's static workspace (no workspace argument)."""
    R, K, V = _step_checks(base, markov, prev0, conf, verify_cost, draft_cost, out, None, status,
                           "dspark_step_static", need_ws=False)
    _check(lib().dspark_step_static(_p(base), _p(markov.A), _p(markov.Bmat), markov.dtype, _p(prev0), R, K, V,
                                    markov.rank, markov._ref, _p(conf), n_sampling, T, num_reqs, _p(verify_cost),
                                    verify_cost.numel(), _p(draft_cost), draft_cost.numel(), _p(out.tokens),
                                    _p(out.surv), _p(out.order), _p(out.sorted_surv), _p(out.b_star),
                                    _p(out.best_obj), _p(out.prefix_len), _p(out.offsets), _p(out.ver_idx),
                                    _p(out.ver_tokens), _p(status), _stream(stream)))


def dspark_schedule(conf, n_sampling: int, T: int, num_reqs: int, verify_cost, draft_cost, out: "StepBuffers",
                    size_conf=None, rule: int = RULE_ARGMAX, tokens=None, status=None, stream=None):
    """Stages 2-5 alone (one kernel) into `out` (its tokens buffer is not touched;
    ver_tokens is filled from `tokens` when given)."""
    R, K = conf.shape
    size_R = -1
    if size_conf is not None:
        if size_conf.dim() != 2 or size_conf.shape[1] != K:
            raise ValueError("dspark_schedule: size_conf must be [R', K]")
        size_R = size_conf.shape[0]
    if tokens is not None and tuple(tokens.shape) != (R, K):
        raise ValueError("dspark_schedule: tokens must be [R, K]")
    _contig(conf, size_conf, verify_cost, draft_cost, tokens)
    _check(lib().dspark_schedule(_p(conf), R, K, _p(size_conf), size_R, rule, n_sampling, T, num_reqs,
                                 _p(verify_cost), verify_cost.numel(), _p(draft_cost), draft_cost.numel(),
                                 _p(tokens), _p(out.surv), _p(out.order), _p(out.sorted_surv), _p(out.b_star),
                                 _p(out.best_obj), _p(out.prefix_len), _p(out.offsets), _p(out.ver_idx),
                                 _p(out.ver_tokens) if tokens is not None else None, _p(status), _stream(stream)))


def dspark_step_sized(base, markov: MarkovHead, prev0, conf, size_conf, rule: int, n_sampling: int, T: int,
                      num_reqs: int, verify_cost, draft_cost, out: "StepBuffers", ws, status=None, stream=None):
    """dspark_step with B sized from `size_conf` ([R', K], e.g. an older step's confidences, or
    None for the current ones) under admission rule `rule`."""
    R, K, V = _step_checks(base, markov, prev0, conf, verify_cost, draft_cost, out, ws, status, "dspark_step_sized")
    size_R = -1                      # -1: size from conf itself
    if size_conf is not None:
        if size_conf.dim() != 2 or size_conf.shape[1] != K or size_conf.dtype != _torch().float32:
            raise ValueError("dspark_step_sized: size_conf must be float32 [R', K]")
        size_R = size_conf.shape[0]
    _contig(size_conf)
    _check(lib().dspark_step_sized(_p(base), _p(markov.A), _p(markov.Bmat), markov.dtype, _p(prev0), R, K, V,
                                   markov.rank, markov._ref, _p(conf), _p(size_conf), size_R, rule, n_sampling, T,
                                   num_reqs, _p(verify_cost), verify_cost.numel(), _p(draft_cost),
                                   draft_cost.numel(), _p(out.tokens), _p(out.surv), _p(out.order),
                                   _p(out.sorted_surv), _p(out.b_star), _p(out.best_obj), _p(out.prefix_len),
                                   _p(out.offsets), _p(out.ver_idx), _p(out.ver_tokens), _p(status), _p(ws),
                                   _ws_bytes(ws), _stream(stream)))


class StepPlan:
    """dspark_step (or dspark_step_sized) with every argument that stays fixed across
    steps -- the head, the scalars, the cost tables, the output buffers, the workspace,
    the status word and the stream -- checked and marshalled once.  A call passes the
    step's own inputs (base, prev0, conf and, when sized, size_conf) and makes one C
    call after cheap shape checks."""

    def __init__(self, markov: MarkovHead, R: int, K: int, n_sampling: int, T: int, num_reqs: int, verify_cost,
                 draft_cost, out: "StepBuffers", ws, status=None, stream=None, rule: int = None):
        torch = _torch()
        dev = markov.A.device
        base0 = torch.empty((R, K, markov.V), dtype=markov.A.dtype, device=dev)
        prev0 = torch.empty(R, dtype=torch.int32, device=dev)
        conf0 = torch.empty((R, K), dtype=torch.float32, device=dev)
        _step_checks(base0, markov, prev0, conf0, verify_cost, draft_cost, out, ws, status, "StepPlan")
        del base0, prev0, conf0
        self.shape = (R, K, markov.V)
        self.rule = rule
        self.markov, self.verify_cost, self.draft_cost, self.out, self.ws, self.status = (
            markov, verify_cost, draft_cost, out, ws, status)
        vp = ctypes.c_void_p
        tail = [vp(_p(out.tokens)), vp(_p(out.surv)), vp(_p(out.order)), vp(_p(out.sorted_surv)),
                vp(_p(out.b_star)), vp(_p(out.best_obj)), vp(_p(out.prefix_len)), vp(_p(out.offsets)),
                vp(_p(out.ver_idx)), vp(_p(out.ver_tokens)), vp(_p(status)), vp(_p(ws)),
                ctypes.c_size_t(_ws_bytes(ws)), vp(_stream(stream))]
        head = [None, vp(_p(markov.A)), vp(_p(markov.Bmat)), ctypes.c_int(markov.dtype), None, ctypes.c_int(R),
                ctypes.c_int(K), ctypes.c_int(markov.V), ctypes.c_int(markov.rank), markov._ref, None]
        scal = [ctypes.c_int(n_sampling), ctypes.c_int(T), ctypes.c_int(num_reqs), vp(_p(verify_cost)),
                ctypes.c_int(verify_cost.numel()), vp(_p(draft_cost)), ctypes.c_int(draft_cost.numel())]
        if rule is None:
            self._fn = lib().dspark_step
            self._args = head + scal + tail
        else:
            self._fn = lib().dspark_step_sized
            self._args = head + [None, None, ctypes.c_int(rule)] + scal + tail

    def __call__(self, base, prev0, conf, size_conf=None):
        if tuple(base.shape) != self.shape or prev0.shape[0] != self.shape[0] or tuple(conf.shape) != self.shape[:2]:
            raise ValueError("StepPlan: input shapes differ from the plan's")
        args = self._args
        args[0] = base.data_ptr()
        args[4] = prev0.data_ptr()
        args[10] = conf.data_ptr()
        if self.rule is not None:
            if size_conf is None:
                args[11], args[12] = None, -1
            else:
                if size_conf.dim() != 2 or size_conf.shape[1] != self.shape[1]:
                    raise ValueError("StepPlan: size_conf must be [R', K]")
                args[11], args[12] = size_conf.data_ptr(), size_conf.shape[0]
        rc = self._fn(*args)
        if rc != 0:
            _check(rc)


def dspark_accept_greedy(ver_tokens, offsets, target, R: int, K: int, accept_len, next_prev0, out_tokens=None,
                         status=None, stream=None):
    """Greedy verification: accepted run, bonus token and next prev0 per request."""
    _contig(ver_tokens, offsets, target, accept_len, next_prev0, out_tokens)
    if offsets.numel() != R + 1 or accept_len.numel() != R or next_prev0.numel() != R \
            or target.numel() < R * K + R or (ver_tokens is not None and ver_tokens.numel() < R * K) \
            or (out_tokens is not None and out_tokens.numel() != R * (K + 1)):
        raise ValueError("dspark_accept_greedy: inconsistent sizes")
    _check(lib().dspark_accept_greedy(_p(ver_tokens), _p(offsets), _p(target), R, K, _p(accept_len),
                                      _p(next_prev0), _p(out_tokens), _p(status), _stream(stream)))


def dspark_set_launch_mode(mode: int):
    """Launch of the persistent kernels: LAUNCH_RESIDENT (plain, default) or LAUNCH_COOPERATIVE."""
    _check(lib().dspark_set_launch_mode(mode))


def dspark_get_launch_mode() -> int:
    return int(lib().dspark_get_launch_mode())


def dspark_set_timing_events(before_chain=None, after_chain=None):
    """Events (torch.cuda.Event or raw handles, already created) that later dspark_step calls on
    this thread set around the chain: the pruned chain kernel's own start and stop, else
    markers before and after the chain's launches."""
    def h(e):
        return None if e is None else (e if isinstance(e, int) else e.cuda_event)
    _check(lib().dspark_set_timing_events(h(before_chain), h(after_chain)))


def dspark_force_monotone(table: np.ndarray) -> np.ndarray:
    """Host-side start-up forcing of a cost table; returns the forced copy."""
    t = np.ascontiguousarray(table, dtype=np.float32).copy()
    _check(lib().dspark_force_monotone(t.ctypes.data_as(ctypes.c_void_p), int(t.size)))
    return t


def dspark_profile_shapes(step, shapes, runs: int = 5, warmup: int = 2, stream=None) -> np.ndarray:
    """Times `step(shape)` (which enqueues one step of that size on the current stream)
    over `shapes`; returns microseconds [len(shapes), runs].  Synchronises."""
    sh = np.ascontiguousarray(shapes, dtype=np.int32)
    out = np.zeros((len(sh), runs), dtype=np.float32)
    failure = []

    def cb(shape, _user, _stream):
        try:
            step(int(shape))
            return 0
        except Exception as exc:        # reported through the library's error path
            failure.append(exc)
            return 1

    fn = SHAPE_FN(cb)
    rc = lib().dspark_profile_shapes(fn, None, sh.ctypes.data_as(ctypes.c_void_p), len(sh), runs, warmup,
                                     out.ctypes.data_as(ctypes.c_void_p), _stream(stream))
    if failure:
        raise failure[0]
    _check(rc)
    return out


def dspark_build_cost_table(shapes, samples_us, graph_max: int, table_len: int) -> np.ndarray:
    """Host-side cost table from profiled runs (median, staircase, continuous tail, forced)."""
    sh = np.ascontiguousarray(shapes, dtype=np.int32)
    smp = np.ascontiguousarray(samples_us, dtype=np.float32)
    if smp.ndim != 2 or smp.shape[0] != len(sh):
        raise ValueError("dspark_build_cost_table: samples must be [len(shapes), runs]")
    table = np.zeros(table_len, dtype=np.float32)
    _check(lib().dspark_build_cost_table(sh.ctypes.data_as(ctypes.c_void_p), len(sh),
                                         smp.ctypes.data_as(ctypes.c_void_p), smp.shape[1], graph_max,
                                         table.ctypes.data_as(ctypes.c_void_p), table_len))
    return table


class StepBuffers:
    """Device output buffers of one step (torch tensors on `device`)."""

    def __init__(self, R: int, K: int, device="cuda"):
        import torch
        i32 = dict(dtype=torch.int32, device=device)
        self.tokens = torch.empty((R, K), **i32)
        self.surv = torch.empty((R, K), dtype=torch.float32, device=device)
        self.order = torch.empty(R * K, **i32)
        self.sorted_surv = torch.empty(R * K, dtype=torch.float32, device=device)
        self.b_star = torch.empty(1, **i32)
        self.best_obj = torch.empty(1, dtype=torch.float64, device=device)
        self.prefix_len = torch.empty(R, **i32)
        self.offsets = torch.empty(R + 1, **i32)
        self.ver_idx = torch.empty(R * K, **i32)
        self.ver_tokens = torch.empty(R * K, **i32)


def workspace(R: int, K: int, V: int, rank: int, dtype: int, device="cuda"):
    import torch
    n = max(dspark_workspace_bytes(R, K, V, rank, dtype), 8)
    # zero-filled once, as the library requires; it then serves calls of any shape up to (R, K)
    return torch.zeros((n + 7) // 8, dtype=torch.int64, device=device)
