"""The segment decomposition behind the context-parallel chunked path, checked in fp64 with the
oracle only (no GPU): per state row the recurrence is affine, so a segment maps its start state
as S_end = S_start M + B, where B is the segment's end state from zero and M is the end state of
the same segment run with v = 0 from the identity.  Chaining the segments and rerunning each from
its chained start must reproduce the direct run exactly (to fp64 rounding)."""
import numpy as np
import pytest

import oracle


def _problem(rng, T, HK, HV, K, V, per_k):
    q = rng.standard_normal((T, HK, K))
    k = rng.standard_normal((T, HK, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, HV, V))
    g = rng.uniform(-2.0, 0.0, (T, HV, K) if per_k else (T, HV))
    beta = rng.uniform(0.0, 1.0, (T, HV))
    h0 = rng.standard_normal((1, HV, V, K)) * 0.3
    return q, k, v, g, beta, h0


@pytest.mark.parametrize("per_k", [False, True])
@pytest.mark.parametrize("cuts", [[0, 64, 128, 192, 205], [0, 37, 100, 101, 205], [0, 205]])
def test_segment_maps_chain_to_the_direct_run(per_k, cuts):
    rng = np.random.default_rng(7 + per_k)
    T, HK, HV, K, V = 205, 1, 2, 8, 4
    q, k, v, g, beta, h0 = _problem(rng, T, HK, HV, K, V, per_k)
    o_ref, f_ref, _ = oracle.recurrent(q, k, v, g, beta, np.array([0, T]), 0.5, h0)

    cu = np.array(cuts, dtype=np.int32)
    P = len(cu) - 1
    # per segment: offset B (zero start) and linear part M (v = 0 from the identity, K state rows)
    _, B, _ = oracle.recurrent(q, k, v, g, beta, cu, 0.5, None)
    eye = np.broadcast_to(np.eye(K), (P, HV, K, K)).copy()
    _, M, _ = oracle.recurrent(q, k, np.zeros((T, HV, K)), g, beta, cu, 0.5, eye)
    # chain: S_0 = h0, S_{s+1} = S_s M_s + B_s
    S = np.zeros((P, HV, V, K))
    S[0] = h0[0]
    for s in range(P - 1):
        S[s + 1] = S[s] @ M[s] + B[s]
    o, fin, _ = oracle.recurrent(q, k, v, g, beta, cu, 0.5, S)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(fin[-1], f_ref[0], rtol=1e-11, atol=1e-12)
    # and the last segment's map applied to its start state is the final state
    np.testing.assert_allclose(S[-1] @ M[-1] + B[-1], f_ref[0], rtol=1e-11, atol=1e-12)
