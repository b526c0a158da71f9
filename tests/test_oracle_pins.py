"""Pins for the CPU oracle: each check ties it to something other than itself.

* hand-worked examples (tests/golden/*.json);
* brute force: dense K x K transition products and the unrolled closed form,
  two formulas different from the oracle's row-wise loop;
* closed forms: T=1 from zero state, beta=0 pure decay, g=0 & beta=0 identity,
  exact retrieval with orthonormal keys and beta=1;
* GQA mapping h // (HV/HK) (FlashQLA PR #1 review commit: "h//grp vs h%Hk");
* negative controls: a pre-update read and an h % HK mapping, planted in a CPU
  re-implementation, must fail the tolerance the GPU tests use;
* the chunk form (oracle/chunk_form.py) equals the token oracle, including the
  adversarial decays where exp(-prefix) would overflow fp32 (cuLA PR #113 review).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import chunk_form
from gated_delta_rule_63_amd import inputs
from _cmp import TOL, max_rel_l2_tokens, rel_l2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["worked_scalar_gate_2x2.json", "worked_per_key_gate_2x2.json"])
def test_hand_worked_example(name):
    d = _golden(name)
    k = np.array(d["k"])[:, None, :]
    q = np.array(d["q"])[:, None, :]
    v = np.array(d["v"])[:, None, :]
    g = np.array(d["g"])
    g = g[:, None] if g.ndim == 1 else g[:, None, :]
    beta = np.array(d["beta"])[:, None]
    T = k.shape[0]
    h0 = np.array(d["initial_state"])[None, None]
    o, fin, _ = oracle.recurrent(q, k, v, g, beta, np.array([0, T]), 1.0, h0)
    np.testing.assert_allclose(o[:, 0], np.array(d["expected_o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0], np.array(d["expected_final_state"]), rtol=0, atol=1e-12)


def _rand_case(rng, T, HK, HV, K, V, per_k, g_lo=-0.5):
    q = rng.standard_normal((T, HK, K))
    k = rng.standard_normal((T, HK, K))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, HV, V))
    g = rng.uniform(g_lo, 0.0, size=(T, HV, K) if per_k else (T, HV))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, HV))))
    return q, k, v, g, beta


def _brute_force(q, k, v, g, beta, h0, scale, grp):
    """S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = scale S_t q_t,
    with dense K x K transition matrices (one sequence)."""
    T, HK, K = q.shape
    HV = v.shape[1]
    o = np.zeros((T, HV, v.shape[2]))
    S_all = []
    for h in range(HV):
        hk = h // grp
        S = h0[h].copy()
        for t in range(T):
            D = np.diag(np.exp(g[t, h])) if g.ndim == 3 else np.exp(g[t, h]) * np.eye(K)
            kt = k[t, hk][:, None]
            M = D @ (np.eye(K) - beta[t, h] * kt @ kt.T)
            S = S @ M + beta[t, h] * v[t, h][:, None] @ kt.T
            o[t, h] = scale * S @ q[t, hk]
        S_all.append(S)
    return o, np.stack(S_all)


def _unrolled_final(k, v, g, beta, h0, grp):
    """S_T = S_0 prod_t M_t + sum_t beta_t v_t k_t^T prod_{s>t} M_s (one sequence)."""
    T, HK, K = k.shape
    HV = v.shape[1]
    out = []
    for h in range(HV):
        hk = h // grp
        Ms = []
        for t in range(T):
            D = np.diag(np.exp(g[t, h])) if g.ndim == 3 else np.exp(g[t, h]) * np.eye(K)
            kt = k[t, hk][:, None]
            Ms.append(D @ (np.eye(K) - beta[t, h] * kt @ kt.T))
        total = h0[h].copy()
        for M in Ms:
            total = total @ M
        for t in range(T):
            tail = np.eye(K)
            for s in range(t + 1, T):
                tail = tail @ Ms[s]
            total = total + beta[t, h] * v[t, h][:, None] @ k[t, hk][None, :] @ tail
        out.append(total)
    return np.stack(out)


@pytest.mark.parametrize("per_k", [False, True])
@pytest.mark.parametrize("HK,HV", [(1, 1), (2, 4), (1, 3)])
def test_brute_force_transition_products(per_k, HK, HV):
    rng = np.random.default_rng(11 + HV + 7 * per_k)
    T, K, V = 7, 5, 6
    q, k, v, g, beta = _rand_case(rng, T, HK, HV, K, V, per_k)
    h0 = rng.standard_normal((1, HV, V, K))
    scale = 0.37
    o, fin, _ = oracle.recurrent(q, k, v, g, beta, np.array([0, T]), scale, h0)
    o_bf, s_bf = _brute_force(q, k, v, g, beta, h0[0], scale, HV // HK)
    np.testing.assert_allclose(o, o_bf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fin[0], s_bf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fin[0], _unrolled_final(k, v, g, beta, h0[0], HV // HK), rtol=0, atol=1e-12)


def test_varlen_equals_separate_sequences():
    rng = np.random.default_rng(5)
    lens = [3, 0, 5, 1]
    T = sum(lens)
    q, k, v, g, beta = _rand_case(rng, T, 2, 4, 6, 5, False)
    cu = np.concatenate([[0], np.cumsum(lens)])
    h0 = rng.standard_normal((4, 4, 5, 6))
    o, fin, _ = oracle.recurrent(q, k, v, g, beta, cu, 0.5, h0)
    for n in range(4):
        s, e = cu[n], cu[n + 1]
        o1, f1, _ = oracle.recurrent(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], np.array([0, e - s]), 0.5, h0[n:n + 1])
        np.testing.assert_array_equal(o[s:e], o1)
        np.testing.assert_array_equal(fin[n], f1[0])
    # an empty sequence is the identity on its state
    np.testing.assert_array_equal(fin[1], h0[1])


def test_single_token_from_zero_state_closed_form():
    rng = np.random.default_rng(6)
    q, k, v, g, beta = _rand_case(rng, 1, 1, 1, 8, 8, False)
    o, fin, _ = oracle.recurrent(q, k, v, g, beta, np.array([0, 1]), 0.25)
    S = beta[0, 0] * np.outer(v[0, 0], k[0, 0])
    np.testing.assert_allclose(fin[0, 0], S, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 0], 0.25 * beta[0, 0] * (k[0, 0] @ q[0, 0]) * v[0, 0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("per_k", [False, True])
def test_beta_zero_is_pure_decay(per_k):
    rng = np.random.default_rng(7)
    T = 9
    q, k, v, g, beta = _rand_case(rng, T, 1, 2, 6, 4, per_k, g_lo=-1.0)
    beta[:] = 0.0
    h0 = rng.standard_normal((1, 2, 4, 6))
    o, fin, st = oracle.recurrent(q, k, v, g, beta, np.array([0, T]), 0.5, h0, want_states=True)
    gam = np.cumsum(g, axis=0)
    for h in range(2):
        for t in range(T):
            St = h0[0, h] * (np.exp(gam[t, h])[None, :] if per_k else np.exp(gam[t, h]))
            np.testing.assert_allclose(st[t, h], St, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(o[t, h], 0.5 * St @ q[t, 0], rtol=1e-12, atol=1e-14)


def test_identity_when_g_and_beta_are_zero():
    rng = np.random.default_rng(8)
    T = 6
    q, k, v, g, beta = _rand_case(rng, T, 1, 1, 6, 4, False)
    g[:] = 0.0
    beta[:] = 0.0
    h0 = rng.standard_normal((1, 1, 4, 6))
    o, fin, _ = oracle.recurrent(q, k, v, g, beta, np.array([0, T]), 0.5, h0)
    np.testing.assert_array_equal(fin, h0)  # bit for bit
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], 0.5 * h0[0, 0] @ q[t, 0], rtol=1e-14, atol=1e-15)


def test_orthonormal_keys_exact_retrieval():
    rng = np.random.default_rng(9)
    K = V = 16
    n = 12
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    keys = Qm[:, :n].T  # n orthonormal keys
    vals = rng.standard_normal((n, V))
    T = 2 * n
    k = np.concatenate([keys, keys])[:, None, :]
    v = np.concatenate([vals, vals * 0 + rng.standard_normal((n, V))])[:, None, :]
    q = k.copy()  # read back the key just written
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    o, fin, _ = oracle.recurrent(q, k, v, g, beta, np.array([0, T]), 0.125)
    # every read returns scale * (the value last written to that key), including overwrites
    np.testing.assert_allclose(o[:, 0], 0.125 * v[:, 0], rtol=0, atol=1e-12)
    for j in range(n):
        np.testing.assert_allclose(fin[0, 0] @ keys[j], v[n + j, 0], rtol=0, atol=1e-12)


def _python_recurrence(q, k, v, g, beta, cu, scale, h0, read_pre_update=False, gqa_mod=False):
    """A CPU re-implementation with switches that plant the two classic mistakes."""
    T, HK, K = q.shape
    HV, V = v.shape[1:]
    grp = HV // HK
    o = np.zeros((T, HV, V))
    for n in range(len(cu) - 1):
        for h in range(HV):
            hk = (h % HK) if gqa_mod else (h // grp)
            S = h0[n, h].copy() if h0 is not None else np.zeros((V, K))
            for t in range(cu[n], cu[n + 1]):
                S = S * (np.exp(g[t, h]) if g.ndim == 2 else np.exp(g[t, h])[None, :])
                pre = scale * S @ q[t, hk]
                nu = beta[t, h] * (v[t, h] - S @ k[t, hk])
                S = S + np.outer(nu, k[t, hk])
                o[t, h] = pre if read_pre_update else scale * S @ q[t, hk]
    return o


def _as_f64(p):
    return [inputs.widen(x) for x in (p.q, p.k, p.v, p.g, p.beta)]


def test_negative_controls_fail_the_tolerance():
    # tiny fp32 workload (2e-3) and a small GQA 2:1 bf16 workload (2e-2)
    p1 = inputs.tiny()
    q, k, v, g, beta = _as_f64(p1)
    o, _, _ = oracle.recurrent(q, k, v, g, beta, p1.cu_seqlens, p1.scale)
    good = _python_recurrence(q, k, v, g, beta, p1.cu_seqlens, p1.scale, None)
    assert max_rel_l2_tokens(good, o, p1.cu_seqlens) < 1e-12
    bad = _python_recurrence(q, k, v, g, beta, p1.cu_seqlens, p1.scale, None, read_pre_update=True)
    assert max_rel_l2_tokens(bad, o, p1.cu_seqlens) > 10 * TOL["f32"]

    p2 = inputs.paged_problem(2, B=4, q_len=3, HK=2, HV=4, K=16, V=8, num_slots=8, pool_dtype="f32")
    q, k, v, g, beta = _as_f64(p2)
    h0 = inputs.widen(p2.pool)[p2.state_indices]
    o, _, _ = oracle.recurrent(q, k, v, g, beta, p2.cu_seqlens, p2.scale, h0)
    good = _python_recurrence(q, k, v, g, beta, p2.cu_seqlens, p2.scale, h0)
    assert max_rel_l2_tokens(good, o, p2.cu_seqlens) < 1e-12
    bad = _python_recurrence(q, k, v, g, beta, p2.cu_seqlens, p2.scale, h0, read_pre_update=True)
    assert max_rel_l2_tokens(bad, o, p2.cu_seqlens) > TOL["bf16"]
    bad = _python_recurrence(q, k, v, g, beta, p2.cu_seqlens, p2.scale, h0, gqa_mod=True)
    assert max_rel_l2_tokens(bad, o, p2.cu_seqlens) > TOL["bf16"]


def test_decode_paged_semantics_follow_the_recurrence():
    p = inputs.paged_problem(3, B=6, q_len=4, HK=1, HV=2, K=8, V=4, num_slots=10, pool_dtype="f32",
                             pad_count=2, ragged=True, commit=True)
    q, k, v, g, beta = _as_f64(p)
    pool = inputs.widen(p.pool)
    res = oracle.decode_paged(q, k, v, g, beta, p.cu_seqlens, p.scale, pool, p.state_indices, want_states=True)
    cu = p.cu_seqlens
    for b in range(p.N):
        s, e = cu[b], cu[b + 1]
        slot = p.state_indices[b]
        if slot < 0:
            assert np.all(np.isnan(res["o"][s:e]))
            assert b not in res["states"]
            continue
        o1, f1, st = oracle.recurrent(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], np.array([0, e - s]),
                                      p.scale, pool[slot][None], want_states=True)
        np.testing.assert_array_equal(res["o"][s:e], o1)
        np.testing.assert_array_equal(res["final"][int(slot)], f1[0])
        np.testing.assert_array_equal(res["states"][b], st)
        np.testing.assert_array_equal(res["states"][b][-1], f1[0])


@pytest.mark.parametrize("per_k", [False, True])
@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunk_form_equals_token_recurrence(per_k, C):
    rng = np.random.default_rng(20 + C + per_k)
    lens = [1, 37, 63, 64, 65, 200] if C != 1 else [1, 37, 65]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = _rand_case(rng, T, 2, 4, 16, 8, per_k, g_lo=-2.0)
    h0 = rng.standard_normal((len(lens), 4, 8, 16))
    o_ref, f_ref, _ = oracle.recurrent(q, k, v, g, beta, cu, 0.25, h0)
    o_c, f_c, _ = chunk_form.chunk_forward(q, k, v, g, beta, cu, 0.25, h0, chunk_size=C)
    np.testing.assert_allclose(o_c, o_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(f_c, f_ref, rtol=0, atol=1e-10)


def test_chunk_form_is_finite_where_exp_minus_prefix_overflows():
    """All gk = -2, beta = 1: inside a 64-token chunk the prefix reaches -128, so a
    factor exp(-prefix) overflows fp32 from the 45th token on; the chunk form uses
    no such factor and must match the token recurrence."""
    p = inputs.kda_overflow_case(T=130, HV=1)
    q, k, v, g, beta = _as_f64(p)
    prefix = np.cumsum(g[:64, 0, 0])
    with np.errstate(over="ignore"):
        inv = np.exp(-prefix.astype(np.float32))
    first_inf = int(np.argmax(~np.isfinite(inv)))
    assert first_inf == 44  # 0-based token index 44, i.e. the 45th token
    o_ref, f_ref, _ = oracle.recurrent(q, k, v, g, beta, p.cu_seqlens, p.scale)
    o_c, f_c, inter = chunk_form.chunk_forward(q, k, v, g, beta, p.cu_seqlens, p.scale, keep_intermediates=True)
    assert np.all(np.isfinite(o_c)) and np.all(np.isfinite(f_c))
    for res in inter.values():
        for key in ("A", "W", "U", "P"):
            assert np.all(np.isfinite(res[key]))
    np.testing.assert_allclose(o_c, o_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(f_c, f_ref, rtol=0, atol=1e-10)


def test_chunk_intermediates_satisfy_their_definitions():
    """A is the inverse of I+L, W/U are A times the scaled keys/values, and C=1
    chunks reduce to one step of the recurrence."""
    rng = np.random.default_rng(31)
    q, k, v, g, beta = _rand_case(rng, 64, 1, 1, 16, 8, False)
    res = chunk_form.chunk_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], np.zeros((8, 16)), 1.0)
    np.testing.assert_allclose((np.eye(64) + res["L"]) @ res["A"], np.eye(64), atol=1e-12)
    assert np.allclose(np.triu(res["L"]), 0.0) and np.allclose(np.triu(res["A"], 1), 0.0)
    # the delta-rule identity: U - W S0^T with S0 = 0 gives the v_new of the token recurrence
    _, _, st = oracle.recurrent(q, k, v, g, beta, np.array([0, 64]), 1.0, want_states=True)
    prev = np.concatenate([np.zeros((1, 8, 16)), st[:-1, 0]])
    for t in range(64):
        nu_t = beta[t, 0] * (v[t, 0] - (prev[t] * math.exp(g[t, 0])) @ k[t, 0])
        np.testing.assert_allclose(res["Nu"][t], nu_t, atol=1e-11)
