"""ORACLE -- test infrastructure only.

A plain, slow, obviously correct CPU implementation of the chain-and-schedule
step.  Only the tests, the package smoke check and the benchmark's CPU-baseline
leg may import it; the product path (the HIP library and its binding) never
does, and shares no code with it.

  * ``chain``          -- stage 1 in plain C, double precision (``chain.c``);
  * ``oracle.sched``   -- stages 2-5 and the cost-table forcing in Python with
                          exact rational arithmetic where the method sums;
  * ``oracle.verify``  -- greedy verification of the allocated drafts (accepted
                          run, bonus token, the next step's prev0).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "chain.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_chain.so")
_lib = None
_lock = threading.Lock()  # tests call the oracle from several host threads at once


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no contraction, no fast-math)."""
    with _lock:
        if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            tmp = f"{_LIB_PATH}.tmp{os.getpid()}"
            subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                                   "-o", tmp, _SRC, "-lm"])
            os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
    build(force=False)
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(_LIB_PATH)
            p = ctypes.c_void_p
            lib.oracle_chain.argtypes = [p, p, p, ctypes.c_int, p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, p, ctypes.c_int, p, p, p, p]
            lib.oracle_chain.restype = ctypes.c_int
            lib.oracle_chain_sample.argtypes = [p, p, p, ctypes.c_int, p, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, p, ctypes.c_int, p, ctypes.c_double,
                                                ctypes.c_uint64, p, p, p]
            lib.oracle_chain_sample.restype = ctypes.c_int
            lib.oracle_philox4x32.argtypes = [p, p, p]
            lib.oracle_philox4x32.restype = None
            _lib = lib
        return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def chain(base, A, Bmat, dtype, prev0, rows=None, forced=None, want_logits=False):
    """Stage 1 (see chain.c).  base [R,K,V], A [V,r], Bmat [r,V] as float32 or bf16 bit patterns (uint16).

    Returns (tokens [n_rows,K] int32, logits [n_rows,K,V] float64 or None, status uint32).
    """
    lib = _load()
    R, K, V = base.shape
    rank = A.shape[1]
    assert A.shape == (V, rank) and Bmat.shape == (rank, V)
    want = np.uint16 if dtype == 1 else np.float32
    base = np.ascontiguousarray(base, dtype=want)
    A = np.ascontiguousarray(A, dtype=want)
    Bmat = np.ascontiguousarray(Bmat, dtype=want)
    prev0 = np.ascontiguousarray(prev0, dtype=np.int32)
    rows = np.arange(R, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    if forced is not None:
        forced = np.ascontiguousarray(forced, dtype=np.int32)
        assert forced.shape == (R, K)
    tokens = np.zeros((len(rows), K), dtype=np.int32)
    logits = np.zeros((len(rows), K, V), dtype=np.float64) if want_logits else None
    status = np.zeros(1, dtype=np.uint32)
    rc = lib.oracle_chain(_ptr(base), _ptr(A), _ptr(Bmat), int(dtype), _ptr(prev0), R, K, V, rank,
                          _ptr(rows), len(rows), _ptr(forced), _ptr(tokens), _ptr(logits), _ptr(status))
    if rc != 0:
        raise ValueError("oracle_chain rejected its arguments")
    return tokens, logits, int(status[0])


def chain_sample(base, A, Bmat, dtype, prev0, temperature, seed, rows=None, forced=None, want_perturbed=False):
    """Stage 1 with probabilistic drafting (see chain.c): token = argmax_v x[v]/temperature + g(seed, r, i, v).

    Returns (tokens [n_rows,K] int32, perturbed values [n_rows,K,V] float64 or None, status)."""
    lib = _load()
    R, K, V = base.shape
    rank = A.shape[1]
    assert A.shape == (V, rank) and Bmat.shape == (rank, V)
    want = np.uint16 if dtype == 1 else np.float32
    base = np.ascontiguousarray(base, dtype=want)
    A = np.ascontiguousarray(A, dtype=want)
    Bmat = np.ascontiguousarray(Bmat, dtype=want)
    prev0 = np.ascontiguousarray(prev0, dtype=np.int32)
    rows = np.arange(R, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    if forced is not None:
        forced = np.ascontiguousarray(forced, dtype=np.int32)
        assert forced.shape == (R, K)
    tokens = np.zeros((len(rows), K), dtype=np.int32)
    pert = np.zeros((len(rows), K, V), dtype=np.float64) if want_perturbed else None
    status = np.zeros(1, dtype=np.uint32)
    rc = lib.oracle_chain_sample(_ptr(base), _ptr(A), _ptr(Bmat), int(dtype), _ptr(prev0), R, K, V, rank,
                                 _ptr(rows), len(rows), _ptr(forced), float(temperature), int(seed),
                                 _ptr(tokens), _ptr(pert), _ptr(status))
    if rc != 0:
        raise ValueError("oracle_chain_sample rejected its arguments")
    return tokens, pert, int(status[0])


def philox4x32(counter, key):
    """The C oracle's Philox4x32-10 (for pinning it against oracle.rng)."""
    lib = _load()
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32(_ptr(c), _ptr(k), _ptr(out))
    return [int(x) for x in out]
