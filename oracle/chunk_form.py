"""Chunked (WY/UT) form of the gated delta rule in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

The pages name the pieces of the chunked algorithm without writing its algebra:
the FlashQLA PR #1 design commit lists "kkt_solve / A / cumsum" as the parts the
recurrent kernel does without, and the attention-gym PR #344 page names the
inter-chunk recurrence's operands (w, u, gated k) and outputs (per-chunk h,
v_new).  The algebra below is derived from the token recurrence (the token
oracle in ``gdr_oracle.c``) by unrolling it over one chunk; it reproduces that
recurrence exactly up to rounding, which ``tests/test_oracle_pins.py`` checks.

For one chunk of C tokens (rows r = 0..C-1, counted from the chunk start, chunks
restart at every sequence start, the last chunk may be short), with start state
S0 [V, K] and the chunk-local cumulative log-decay gamma_r = sum_{s<=r} g_s
(per channel for the per-K gate):

  L[r, j] = beta_r * sum_c k_rc k_jc exp(gamma_rc - gamma_jc)      r > j, else 0
  A       = (I + L)^-1                                              unit lower-triangular
  U       = A diag(beta) V
  W       = A diag(beta) (K * exp(gamma))
  Nu      = U - W S0^T                                              (rows = v_new_r)
  S_C     = S0 * exp(gamma_last) + Nu^T (K * exp(gamma_last - gamma))
  P[r, j] = sum_c q_rc k_jc exp(gamma_rc - gamma_jc)                r >= j, else 0
  O       = scale * ((Q * exp(gamma)) S0^T + P Nu)

Every exponent used is (later - earlier) <= 0 or gamma <= 0, so no factor above
exceeds 1: this is the overflow-free form the cuLA PR #113 review asks for (an
exp(-prefix) factor overflows fp32 once the 64-token prefix passes about -88).
The scalar gate is the per-K case with every channel equal.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _decay_matrix(gam_r: np.ndarray, gam_j: np.ndarray, inclusive: bool) -> np.ndarray:
    """D[r, j, c] = exp(gam_r[r, c] - gam_j[j, c]) on r > j (or r >= j), 0 elsewhere.
    The exponent is masked before exp so the upper triangle never overflows."""
    C = gam_r.shape[0]
    r = np.arange(C)[:, None]
    j = np.arange(C)[None, :]
    keep = (r >= j) if inclusive else (r > j)
    diff = gam_r[:, None, :] - gam_j[None, :, :]
    diff = np.where(keep[:, :, None], diff, -np.inf)
    return np.exp(diff)


def chunk_step(q, k, v, g, beta, S0, scale: float):
    """One chunk, one head.  q, k [C, K]; v [C, V]; g [C] or [C, K]; beta [C]; S0 [V, K].

    Returns a dict with gamma, L, A, U, W, Nu, S_end, P, O (all float64)."""
    q, k, v, g, beta, S0 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, S0))
    C, K = k.shape
    gam = np.cumsum(g, axis=0)
    gamk = gam if gam.ndim == 2 else np.repeat(gam[:, None], K, axis=1)  # [C, K]
    Dl = _decay_matrix(gamk, gamk, inclusive=False)
    L = beta[:, None] * np.einsum("rc,jc,rjc->rj", k, k, Dl)
    A = np.linalg.inv(np.eye(C) + L)
    A = np.tril(A)  # exact zeros above the diagonal (inverse of a lower-triangular matrix)
    U = A @ (beta[:, None] * v)
    W = A @ (beta[:, None] * (k * np.exp(gamk)))
    Nu = U - W @ S0.T
    last = gamk[C - 1]
    S_end = S0 * np.exp(last)[None, :] + Nu.T @ (k * np.exp(last[None, :] - gamk))
    Dp = _decay_matrix(gamk, gamk, inclusive=True)
    P = np.einsum("rc,jc,rjc->rj", q, k, Dp)
    O = scale * ((q * np.exp(gamk)) @ S0.T + P @ Nu)
    return {"gamma": gam, "L": L, "A": A, "U": U, "W": W, "Nu": Nu, "S_end": S_end, "P": P, "O": O}


def chunk_forward(q, k, v, g, beta, cu_seqlens, scale: float, initial_state=None,
                  chunk_size: int = 64, keep_intermediates: bool = False):
    """Whole packed-varlen problem through the chunk form.

    Same layouts as the token oracle: q, k [T, HK, K]; v [T, HV, V]; g [T, HV] or
    [T, HV, K]; beta [T, HV]; initial_state [N, HV, V, K] or None.
    Returns (o [T, HV, V], final [N, HV, V, K], inter) where inter (if asked) maps
    (chunk_index, head) -> chunk_step dict plus "S0"; chunks are numbered in
    sequence order, ceil(len / chunk_size) per sequence.
    """
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    grp = HV // HK
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    o = np.zeros((T, HV, V))
    fin = np.zeros((N, HV, V, K))
    inter = {} if keep_intermediates else None
    cidx = 0
    for n in range(N):
        bos, eos = int(cu[n]), int(cu[n + 1])
        nchunks = (eos - bos + chunk_size - 1) // chunk_size
        for h in range(HV):
            hk = h // grp
            S = np.zeros((V, K)) if initial_state is None else np.asarray(initial_state[n, h], dtype=np.float64)
            for c in range(nchunks):
                s, e = bos + c * chunk_size, min(eos, bos + (c + 1) * chunk_size)
                res = chunk_step(q[s:e, hk], k[s:e, hk], v[s:e, h], g[s:e, h], beta[s:e, h], S, scale)
                o[s:e, h] = res["O"]
                if inter is not None:
                    res["S0"] = S
                    inter[(cidx + c, h)] = res
                S = res["S_end"]
            fin[n, h] = S
        cidx += nchunks
    return o, fin, inter


def chunk_table(cu_seqlens, chunk_size: int = 64):
    """(seq, start, length) of every chunk, numbered in sequence order."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = []
    for n in range(cu.shape[0] - 1):
        bos, eos = int(cu[n]), int(cu[n + 1])
        for s in range(bos, eos, chunk_size):
            out.append((n, s, min(chunk_size, eos - s)))
    return out


def max_chunks(T: int, N: int, chunk_size: int = 64) -> Optional[int]:
    return T // chunk_size + N
