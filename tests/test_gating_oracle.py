"""Pins for the gating oracle (oracle/gating.py), each against something other than itself.

* a hand-worked example (tests/golden/worked_gating.json);
* library routines with different formulas: numpy.logaddexp for softplus below the
  threshold, scipy.special.expit for the sigmoid;
* closed forms and invariants: softplus(0) = ln 2, the pass-through above 20, g <= 0,
  sigmoid(x) + sigmoid(-x) = 1, unit length and direction of the normalised rows, the
  length sqrt(|x|^2 / (|x|^2 + eps)) with eps > 0, scale invariance;
* negative controls: feeding the recurrence raw a as the decay, or unnormalised q/k,
  moves its outputs far outside the tolerance the GPU tests use, so the gated parity
  tests can tell a skipped step from a correct one.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import gating
from gated_delta_rule_63_amd import inputs
from _cmp import TOL, max_rel_l2_tokens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_gating.json")


def test_hand_worked_example():
    with open(GOLDEN) as f:
        d = json.load(f)
    g = gating.decay(np.array(d["a"]), np.array(d["A_log"]), np.array(d["dt_bias"]))
    np.testing.assert_allclose(g, np.array(d["expected_g"]), rtol=1e-15, atol=0)
    np.testing.assert_allclose(gating.beta_gate(np.array(d["b"]), False), np.array(d["expected_beta"]),
                               rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(gating.beta_gate(np.array(d["b"]), True), np.array(d["expected_beta_neg_eigval"]),
                               rtol=1e-15, atol=1e-16)
    qn, kn, g2, b2 = gating.gated_inputs(np.array(d["q"]), np.array(d["k"]), np.array(d["a"]), np.array(d["b"]),
                                         np.array(d["A_log"]), np.array(d["dt_bias"]), 0.0, True, False)
    np.testing.assert_allclose(qn, np.array(d["expected_q"]), rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(kn, np.array(d["expected_k"]), rtol=1e-15, atol=1e-16)
    np.testing.assert_array_equal(g2, g)
    e = d["eps_case"]
    np.testing.assert_allclose(gating.l2norm(np.array(e["x"]), e["eps"]), np.array(e["expected"]), rtol=1e-15)


def test_softplus_matches_logaddexp_below_threshold():
    x = np.concatenate([np.linspace(-40.0, 20.0, 6001), [-1e-300, 0.0, 1e-300, 19.999999]])
    np.testing.assert_allclose(gating.softplus(x), np.logaddexp(0.0, x), rtol=1e-14, atol=0)
    assert gating.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-16)


def test_softplus_passes_through_above_threshold():
    x = np.array([20.0 + 1e-12, 20.5, 25.0, 88.0, 1e6])
    np.testing.assert_array_equal(gating.softplus(x), x)
    # at exactly 20 the smooth branch applies; the two branches differ there by ~e^-20
    assert gating.softplus(20.0) == pytest.approx(20.0 + math.log1p(math.exp(-20.0)), rel=1e-15)
    assert abs(gating.softplus(20.0) - 20.0) < 3e-9


def test_sigmoid_matches_expit_and_symmetry():
    x = np.linspace(-30.0, 30.0, 1201)
    np.testing.assert_allclose(gating.sigmoid(x), expit(x), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(gating.sigmoid(x) + gating.sigmoid(-x), 1.0, rtol=1e-15)
    assert gating.sigmoid(0.0) == 0.5
    b = gating.beta_gate(x, True)
    assert np.all((b > 0) & (b < 2)) and np.array_equal(b, 2 * gating.beta_gate(x, False))


def test_decay_closed_forms():
    rng = np.random.default_rng(11)
    a = rng.normal(0, 3, (50, 4))
    A_log = rng.normal(0, 1, 4)
    dt = rng.normal(0, 2, 4)
    g = gating.decay(a, A_log, dt)
    assert np.all(g <= 0) and np.all(np.isfinite(g))
    x = a + dt[None, :]
    below = x <= 20.0
    ref = -np.exp(A_log)[None, :] * np.logaddexp(0.0, x)
    np.testing.assert_allclose(g[below], ref[below], rtol=1e-14)
    # a above the threshold: exactly linear in a
    a_hi = np.full((3, 4), 30.0)
    assert np.all(30.0 + dt > 20.0)
    np.testing.assert_allclose(gating.decay(a_hi, A_log, dt),
                               np.broadcast_to(-np.exp(A_log)[None, :] * (30.0 + dt[None, :]), (3, 4)), rtol=1e-15)
    # monotone: a larger a decays more
    assert np.all(np.diff(gating.decay(np.linspace(-10, 30, 81)[:, None], A_log[:1], dt[:1])[:, 0]) < 0)


def test_l2norm_invariants():
    rng = np.random.default_rng(12)
    x = rng.normal(0, 1, (40, 3, 128)) * rng.uniform(0.01, 100, (40, 3, 1))
    y = gating.l2norm(x, 0.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-14)
    # parallel to x: y * |x| == x
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-13, atol=1e-13)
    # scale invariance without eps
    np.testing.assert_allclose(gating.l2norm(7.5 * x, 0.0), y, rtol=1e-14, atol=1e-16)
    # with eps: length sqrt(n2 / (n2 + eps))
    eps = 0.3
    n2 = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.linalg.norm(gating.l2norm(x, eps), axis=-1), np.sqrt(n2 / (n2 + eps)), rtol=1e-14)
    # the zero row stays zero with eps > 0
    assert np.array_equal(gating.l2norm(np.zeros((1, 128)), 1e-6), np.zeros((1, 128)))


def _gated_decode(p, r, skip_gate=False, skip_norm=False):
    qn, kn, g, beta = gating.gated_inputs(inputs.widen(r.q), inputs.widen(r.k), inputs.widen(r.a),
                                          inputs.widen(r.b), r.A_log, r.dt_bias, r.eps, r.qk_l2norm,
                                          r.allow_neg_eigval)
    if skip_gate:
        g = np.minimum(inputs.widen(r.a), 0.0)  # the raw input taken as an (already valid) log decay
    if skip_norm:
        qn, kn = inputs.widen(r.q), inputs.widen(r.k)
    return oracle.decode_paged(qn, kn, inputs.widen(p.v), g, beta, p.cu_seqlens, p.scale,
                               inputs.widen(p.pool), p.state_indices)


def test_negative_controls_fail_the_tolerance():
    p = inputs.paged_problem(21, B=6, q_len=4, HK=2, HV=4, K=32, V=16, num_slots=8, pool_dtype="f32")
    r = inputs.raw_gating(22, p.T, p.HK, p.HV, p.K, io_dtype=p.io_dtype)
    good = _gated_decode(p, r)["o"]
    for kw in ({"skip_gate": True}, {"skip_norm": True}):
        bad = _gated_decode(p, r, **kw)["o"]
        assert max_rel_l2_tokens(bad, good, p.cu_seqlens) > 10 * TOL["bf16"], kw
    # beta doubled is also told apart
    r2 = inputs.raw_gating(22, p.T, p.HK, p.HV, p.K, io_dtype=p.io_dtype, allow_neg_eigval=True)
    assert max_rel_l2_tokens(_gated_decode(p, r2)["o"], good, p.cu_seqlens) > TOL["bf16"]


def test_generator_exercises_both_softplus_branches():
    r = inputs.raw_gating(5, 4096, 2, 8, 64)
    x = inputs.widen(r.a) + r.dt_bias[None, :]
    assert np.any(x > 20.0) and np.any(x < 20.0)
