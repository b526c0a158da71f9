"""CPU oracle for the fused KDA decode front -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this module; the product path never does.

What it computes (tokenspeed PR #834 "[WIP] perf(k3): optimize decode": the commit that
rewrites the single-launch KDA decode -- a causal convolution with SiLU, the gate
projection, q/k l2 normalisation and the delta-rule recurrence against the paged fp32
state -- and the commit that folds rmsnorm(o) * w * sigmoid(gate) into its epilogue).
The page names these steps but not their formulas; the readings taken here are:

  conv     each channel c of q, k and v (raw projections) runs a causal depthwise
           convolution of width W over its own history:
               y_t[c] = silu(bias[c] + sum_{i<W} w[c][i] * x_{t-(W-1)+i}[c])
           where x_{t-j} for tokens before the first one of the call come from the
           per-slot window (the W-1 latest raw inputs, oldest first); silu(z) = z sigmoid(z).
           After the call the window holds the W-1 latest raw inputs.
  gate     a low-rank projection of a per-token gate input a_t [R] to one value per key
           channel of each value head, then the decay of the gating front applied per channel:
               gk[t,h,c] = -exp(A_log[h]) * softplus((W_g a_t)[h*K + c] + dt_bias[h*K + c])
           softplus with threshold 20 (as the gating front).
  norm     q and k after the convolution are l2-normalised per (token, head) with an eps.
  beta     sigmoid(b[t,h]).
  epilogue optional: o <- o / sqrt(mean_v o^2 + eps) * w[v] * sigmoid(z[t,h,v]).

The recurrence itself is ``oracle.decode_paged`` with the per-key-channel gate.  Everything
is float64 numpy following the definitions; inputs are the exact values handed to the GPU.
The pins live in ``tests/test_kda_front_oracle.py``.
"""
from __future__ import annotations

import numpy as np

from . import decode_paged
from .gating import l2norm, sigmoid, softplus


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def conv_silu(x, window, weight, bias=None):
    """Causal depthwise convolution with SiLU over one sequence.

    x [L, C] raw inputs; window [C, W-1] the W-1 previous raw inputs, oldest first;
    weight [C, W] taps, oldest first; bias [C] or None.
    Returns (y [L, C], new_window [C, W-1]).
    """
    x = np.asarray(x, dtype=np.float64)
    window = np.asarray(window, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.float64)
    L, C = x.shape
    W = weight.shape[1]
    assert window.shape == (C, W - 1)
    hist = np.concatenate([window.T, x], axis=0)          # [W-1+L, C], oldest first
    y = np.empty((L, C), dtype=np.float64)
    for t in range(L):
        z = np.sum(hist[t:t + W].T * weight, axis=1)
        if bias is not None:
            z = z + np.asarray(bias, dtype=np.float64)
        y[t] = silu(z)
    return y, np.ascontiguousarray(hist[L:].T)


def kda_gate(gate_in, gate_weight, A_log, dt_bias, HV: int, K: int):
    """Per-key-channel log decay gk [T, HV, K] from gate_in [T, R], gate_weight [HV*K, R],
    A_log [HV], dt_bias [HV*K]."""
    raw = np.asarray(gate_in, dtype=np.float64) @ np.asarray(gate_weight, dtype=np.float64).T
    x = raw + np.asarray(dt_bias, dtype=np.float64)[None, :]
    T = x.shape[0]
    return -np.exp(np.asarray(A_log, dtype=np.float64))[None, :, None] * softplus(x).reshape(T, HV, K)


def gated_rmsnorm(o, weight, z, eps: float):
    """o [..., V] / sqrt(mean over V of o^2 + eps) * weight [V] * sigmoid(z [..., V])."""
    o = np.asarray(o, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + float(eps)) * np.asarray(weight, dtype=np.float64) * sigmoid(z)


def kda_decode_front(q, k, v, conv_weight, conv_bias, conv_state, gate_in, gate_weight, A_log, dt_bias, b,
                     cu_seqlens, scale: float, pool, state_indices, l2_eps: float,
                     norm_weight=None, norm_gate=None, norm_eps: float = 0.0):
    """The fused front over a paged batch (one key head per value head: HK == HV).

    q, k [T, H, K] and v [T, H, V] raw projections; conv_weight [C, W], conv_bias [C] or None,
    conv_state [slots, C, W-1] with C = 2*H*K + H*V channels in the order q | k | v (head-major);
    gate_in [T, R], gate_weight [H*K, R], A_log [H], dt_bias [H*K], b [T, H]; pool and
    state_indices as ``decode_paged`` (a negative index skips the sequence).
    Returns a dict: "o" [T, H, V] (NaN on skipped rows), "final" {slot: [H, V, K]},
    "conv" {slot: [C, W-1]} (the window after the sequence), and the intermediates "q", "k",
    "v", "g", "beta" (NaN rows for skipped sequences).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    T, H, K = q.shape
    V = v.shape[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    idx = np.asarray(state_indices, dtype=np.int64)
    qc = np.full_like(q, np.nan)
    kc = np.full_like(k, np.nan)
    vc = np.full_like(v, np.nan)
    conv_out = {}
    for n in range(idx.shape[0]):
        slot = int(idx[n])
        if slot < 0:
            continue
        s, e = int(cu[n]), int(cu[n + 1])
        x = np.concatenate([q[s:e].reshape(e - s, H * K), k[s:e].reshape(e - s, H * K),
                            v[s:e].reshape(e - s, H * V)], axis=1)
        y, win = conv_silu(x, conv_state[slot], conv_weight, conv_bias)
        qc[s:e] = y[:, :H * K].reshape(e - s, H, K)
        kc[s:e] = y[:, H * K:2 * H * K].reshape(e - s, H, K)
        vc[s:e] = y[:, 2 * H * K:].reshape(e - s, H, V)
        conv_out[slot] = win
    qn = l2norm(qc, l2_eps)
    kn = l2norm(kc, l2_eps)
    g = kda_gate(gate_in, gate_weight, A_log, dt_bias, H, K)
    beta = sigmoid(b)
    # the recurrence reads only the rows of active sequences; zero the others so no NaN enters it
    act_rows = np.zeros(T, dtype=bool)
    for n in range(idx.shape[0]):
        if idx[n] >= 0:
            act_rows[int(cu[n]):int(cu[n + 1])] = True
    z = lambda a: np.where(act_rows.reshape((T,) + (1,) * (a.ndim - 1)), a, 0.0)
    ref = decode_paged(z(qn), z(kn), z(vc), g, beta, cu, scale, pool, idx)
    o = ref["o"]
    if norm_weight is not None:
        o = gated_rmsnorm(o, norm_weight, norm_gate, norm_eps)
    return {"o": o, "final": ref["final"], "conv": conv_out, "q": qn, "k": kn, "v": vc, "g": g, "beta": beta}
