"""Comparison rules shared by the tests.

relL2 per (sequence, head) slice: ||x - ref||_2 / max(||ref||_2, 1e-6 * sqrt(numel)).
The maximum over slices must stay within the tolerance: 2e-3 for fp32 I/O, 2e-2 for
bf16 I/O (the bar set for this path).  Per slice is the strict reading: one bad head
or one short sequence cannot hide in a global norm.
"""
import numpy as np

TOL = {"f32": 2e-3, "bf16": 2e-2}


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.linalg.norm((x - ref).ravel()))
    den = max(float(np.linalg.norm(ref.ravel())), 1e-6 * np.sqrt(max(ref.size, 1)))
    return num / den


def max_rel_l2_tokens(x, ref, cu_seqlens) -> float:
    """x, ref [T, H, D]: max over (sequence, head) slices of relL2."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    worst = 0.0
    for n in range(cu.shape[0] - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        if e <= s:
            continue
        for h in range(ref.shape[1]):
            worst = max(worst, rel_l2(x[s:e, h], ref[s:e, h]))
    return worst


def max_rel_l2_states(x, ref) -> float:
    """x, ref [..., V, K]: max over leading slices."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lead = ref.shape[:-2]
    xs = x.reshape((-1,) + ref.shape[-2:])
    rs = ref.reshape((-1,) + ref.shape[-2:])
    return max((rel_l2(a, b) for a, b in zip(xs, rs)), default=0.0) if len(lead) else rel_l2(x, ref)


def max_rel_l2_slices(x, ref, nd: int) -> float:
    """Max relL2 over every slice formed by the last ``nd`` axes (all leading indices), vectorised;
    the same per-slice rule as rel_l2."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape
    inner = int(np.prod(ref.shape[-nd:])) if nd else 1
    xs = x.reshape(-1, inner)
    rs = ref.reshape(-1, inner)
    if xs.shape[0] == 0:
        return 0.0
    num = np.linalg.norm(xs - rs, axis=1)
    den = np.maximum(np.linalg.norm(rs, axis=1), 1e-6 * np.sqrt(max(inner, 1)))
    return float(np.max(num / den))
