"""CPU oracle for the gating front of the recurrence -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this module; the product path never does.

What it computes (FlashQLA PR #1 "Fused recurrent GDN decode + SGLang DFlash verify
kernel (TileLang, SM90)": the host-gating wrapper commit, the in-kernel gated verify
commit and the pull-request description):

    g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
    beta[t,h] = sigmoid(b[t,h])            (times 2 when negative eigenvalues are allowed)
    q, k      <- l2-normalised per (token, key head) over the K channels

softplus is the one with beta 1 and threshold 20 (the description's "softplus 1.0/20.0"):
inputs above 20 pass through unchanged.  The pages name the l2 normalisation but give no
epsilon; here x / sqrt(sum x^2 + eps) with eps an explicit argument.

Everything is float64 numpy, element by element as the definitions read; inputs are the
exact values handed to the GPU (bf16 widened exactly).  The pins live in
``tests/test_gating_oracle.py``.
"""
from __future__ import annotations

import numpy as np

SOFTPLUS_THRESHOLD = 20.0


def softplus(x):
    """log(1 + e^x), and x itself above the threshold 20."""
    x = np.asarray(x, dtype=np.float64)
    below = np.minimum(x, SOFTPLUS_THRESHOLD)  # keep exp() finite on the branch not taken
    return np.where(x > SOFTPLUS_THRESHOLD, x, np.log1p(np.exp(below)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def decay(a, A_log, dt_bias):
    """Natural-log decay g [T, HV] from the raw input a [T, HV] and per-head A_log, dt_bias [HV]."""
    a = np.asarray(a, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    return -np.exp(A_log)[None, :] * softplus(a + dt_bias[None, :])


def beta_gate(b, allow_neg_eigval: bool):
    """beta [T, HV] from the raw input b [T, HV]."""
    s = sigmoid(b)
    return 2.0 * s if allow_neg_eigval else s


def l2norm(x, eps: float):
    """x / sqrt(sum over the last axis of x^2 + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + float(eps))


def gated_inputs(q, k, a, b, A_log, dt_bias, eps: float, qk_l2norm: bool, allow_neg_eigval: bool):
    """(q, k, g, beta) as the recurrence consumes them."""
    qn = l2norm(q, eps) if qk_l2norm else np.asarray(q, dtype=np.float64)
    kn = l2norm(k, eps) if qk_l2norm else np.asarray(k, dtype=np.float64)
    return qn, kn, decay(a, A_log, dt_bias), beta_gate(b, allow_neg_eigval)
