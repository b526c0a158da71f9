"""CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports it, and it imports nothing from the product path.

Contents
--------
* ``recurrent``       token-by-token fp64 recurrence (C, OpenMP; ``gdr_oracle.c``).
* ``decode_paged``    the paged decode / speculative-verify semantics written out
                      on top of ``recurrent`` (slot gather, -1 skip, commit,
                      per-token intermediate states).
* ``chunk_form``      the chunk-64 WY/UT algebra in numpy fp64 (module of its own).
* ``gating``          the gating front: decay from (a, A_log, dt_bias) through softplus,
                      beta through the sigmoid, q/k l2 normalisation (numpy fp64).

Every function takes float64 numpy arrays (widen bf16 inputs exactly before
calling) and returns float64.  Pins: see ``tests/test_oracle_pins.py``
(brute-force transition products, closed forms, invariants, negative controls,
chunked == recurrent).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdr_oracle_recurrent.restype = ctypes.c_int
        lib.gdr_oracle_recurrent.argtypes = [
            ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_double,
            dp, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int32]
        lib.gdr_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    return a


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(q, k, v, g, beta, cu_seqlens, scale: float, initial_state=None,
              want_states: bool = False, threads: Optional[int] = None):
    """Token-by-token gated delta rule in fp64.

    q, k [T, HK, K]; v [T, HV, V]; g [T, HV] (scalar gate) or [T, HV, K] (per-K gate);
    beta [T, HV]; cu_seqlens int [N+1]; initial_state [N, HV, V, K] or None (zeros).
    Returns (o [T, HV, V], final_state [N, HV, V, K], states [T, HV, V, K] or None).
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    per_k = 1 if g.ndim == 3 else 0
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = cu.shape[0] - 1
    assert k.shape == q.shape and v.shape[0] == T and beta.shape == (T, HV)
    assert int(cu[-1]) == T and int(cu[0]) == 0
    h0 = None if initial_state is None else _f64(initial_state)
    if h0 is not None:
        assert h0.shape == (N, HV, V, K)
    o = np.zeros((T, HV, V), dtype=np.float64)
    fin = np.zeros((N, HV, V, K), dtype=np.float64)
    st = np.zeros((T, HV, V, K), dtype=np.float64) if want_states else None
    rc = _load().gdr_oracle_recurrent(
        T, N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), HK, HV, K, V, per_k,
        float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
        _ptr(fin), _ptr(st), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the shapes (HV % HK != 0 or a non-positive size)")
    return o, fin, st


def decode_paged(q, k, v, g, beta, cu_seqlens, scale: float, pool, state_indices,
                 want_states: bool = False, threads: Optional[int] = None):
    """Paged decode / speculative verify, written out on top of ``recurrent``.

    Semantics (FlashQLA PR #1, verify-kernel and deployment-facts commits):
    sequence b reads its start state from pool[state_indices[b]]; a negative index
    means a padded sequence that is skipped entirely (nothing read or written).
    Returns a dict with
      "o"        [T, HV, V] expected outputs, NaN on rows of skipped sequences;
      "final"    {slot: [HV, V, K]} state after the sequence's last token
                 (what a commit writes back);
      "states"   {b: [L_b, HV, V, K]} post-update state after every token
                 (what the per-token intermediate buffer receives), if asked.
    ``pool`` is only indexed at the active slots, so a caller may pass any object
    supporting ``pool[slot]`` (e.g. a dict of float64 arrays).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    idx = np.asarray(state_indices, dtype=np.int64)
    B = idx.shape[0]
    T = q.shape[0]
    HV, V = v.shape[1], v.shape[2]
    o = np.full((T, HV, V), np.nan, dtype=np.float64)
    active = [b for b in range(B) if idx[b] >= 0]
    final, states = {}, {}
    if not active:
        return {"o": o, "final": final, "states": states}
    # pack the active sequences into one varlen problem
    rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in active]) if active else np.zeros(0, np.int64)
    lens = np.array([cu[b + 1] - cu[b] for b in active], dtype=np.int64)
    sub_cu = np.zeros(len(active) + 1, dtype=np.int32)
    sub_cu[1:] = np.cumsum(lens)
    h0 = np.stack([_f64(pool[int(idx[b])]) for b in active])
    so, sfin, sst = recurrent(_f64(q)[rows], _f64(k)[rows], _f64(v)[rows], _f64(g)[rows],
                              _f64(beta)[rows], sub_cu, scale, h0, want_states, threads)
    o[rows] = so
    for j, b in enumerate(active):
        final[int(idx[b])] = sfin[j]
        if want_states:
            states[b] = sst[sub_cu[j]:sub_cu[j + 1]]
    return {"o": o, "final": final, "states": states}
