"""Pins of the KDA decode-front oracle (oracle/kda_front.py) against facts from outside it:
a library convolution, library sigmoid / softplus forms, closed forms of the gate and the gated
RMSNorm, the streaming property of the causal convolution, a hand-worked end-to-end example
(tests/golden/worked_kda_front.json) and negative controls.  No GPU."""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import kda_front

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_kda_front.json")


def test_conv_matches_numpy_convolve_and_expit_silu():
    rng = np.random.default_rng(0)
    for W in (1, 2, 3, 4):
        L, C = 7, 5
        x = rng.standard_normal((L, C))
        win = rng.standard_normal((C, W - 1))
        w = rng.standard_normal((C, W))
        bias = rng.standard_normal(C)
        y, _ = kda_front.conv_silu(x, win, w, bias)
        for c in range(C):
            hist = np.concatenate([win[c], x[:, c]])
            # np.convolve flips its second argument: taps reversed give the causal correlation
            z = np.convolve(hist, w[c, ::-1], mode="valid") + bias[c]
            np.testing.assert_allclose(y[:, c], z * expit(z), rtol=1e-13, atol=1e-13)


def test_conv_streaming_equals_whole_sequence_and_window_holds_latest_inputs():
    rng = np.random.default_rng(1)
    for W in (2, 3, 4):
        L, C = 9, 4
        x = rng.standard_normal((L, C))
        win0 = rng.standard_normal((C, W - 1))
        w = rng.standard_normal((C, W))
        y_all, win_all = kda_front.conv_silu(x, win0, w)
        win = win0
        ys = []
        for t in range(L):
            yt, win = kda_front.conv_silu(x[t:t + 1], win, w)
            ys.append(yt[0])
        np.testing.assert_array_equal(np.stack(ys), y_all)
        np.testing.assert_array_equal(win, win_all)
        np.testing.assert_array_equal(win_all, x[L - (W - 1):].T)
        # fewer tokens than the window: part of the old window survives
        _, w1 = kda_front.conv_silu(x[:1], win0, w)
        np.testing.assert_array_equal(w1, np.concatenate([win0[:, 1:], x[:1].T], axis=1))


def test_gate_closed_forms_and_head_layout():
    H, K, R = 3, 4, 5
    rng = np.random.default_rng(2)
    A_log = np.log(rng.uniform(1.0, 8.0, H))
    dt = rng.uniform(-6.0, 2.0, H * K)
    # a zero projection leaves -exp(A_log) softplus(dt_bias), softplus = logaddexp(0, x) below 20
    g0 = kda_front.kda_gate(rng.standard_normal((2, R)), np.zeros((H * K, R)), A_log, dt, H, K)
    want = -np.exp(A_log)[:, None] * np.logaddexp(0.0, dt.reshape(H, K))
    np.testing.assert_allclose(g0, np.broadcast_to(want, g0.shape), rtol=1e-14)
    # one-hot projection rows: row h*K + c of the weight feeds head h, channel c
    wg = np.zeros((H * K, R))
    wg[1 * K + 2, 3] = 1.0
    a = np.zeros((1, R))
    a[0, 3] = 7.0
    g1 = kda_front.kda_gate(a, wg, np.zeros(H), np.zeros(H * K), H, K)
    assert g1[0, 1, 2] == pytest.approx(-np.logaddexp(0.0, 7.0), rel=1e-14)
    assert np.all(g1[0][np.arange(H)[:, None] * K + np.arange(K) != 1 * K + 2] == -np.log(2.0))
    # above the threshold the input passes through exactly; g <= 0 and falls as the input grows
    big = kda_front.kda_gate(np.array([[1.0]]), np.array([[25.0]]), np.array([0.0]), np.array([0.5]), 1, 1)
    assert big[0, 0, 0] == -25.5
    xs = np.linspace(-30, 30, 61)[:, None]
    gs = kda_front.kda_gate(xs, np.ones((1, 1)), np.array([0.3]), np.zeros(1), 1, 1)[:, 0, 0]
    assert np.all(gs <= 0) and np.all(np.diff(gs) < 0)


def test_gated_rmsnorm_closed_forms():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((4, 3, 16))
    w = rng.uniform(0.5, 2.0, 16)
    z = rng.standard_normal((4, 3, 16))
    out = kda_front.gated_rmsnorm(o, w, z, 0.0)
    # scale invariance with eps = 0
    np.testing.assert_allclose(kda_front.gated_rmsnorm(7.5 * o, w, z, 0.0), out, rtol=1e-13)
    # unit weight, gate far open: unit root-mean-square
    unit = kda_front.gated_rmsnorm(o, np.ones(16), np.full_like(z, 60.0), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(unit ** 2, axis=-1)), 1.0, rtol=1e-13)
    # a constant vector c: c / sqrt(c^2 + eps) times w times sigmoid(0) = 1/2
    c = np.full((1, 16), -3.0)
    got = kda_front.gated_rmsnorm(c, w, np.zeros((1, 16)), 7.0)
    np.testing.assert_allclose(got[0], -3.0 / 4.0 * w * 0.5, rtol=1e-14)


def _golden_front(fx, **over):
    kw = dict(q=np.array(fx["q"]), k=np.array(fx["k"]), v=np.array(fx["v"]),
              conv_weight=np.array(fx["conv_weight"]), conv_bias=None, conv_state=np.array(fx["conv_state"]),
              gate_in=np.array(fx["gate_in"]), gate_weight=np.array(fx["gate_weight"]), A_log=np.array(fx["A_log"]),
              dt_bias=np.array(fx["dt_bias"]), b=np.array(fx["b"]), cu_seqlens=np.array(fx["cu_seqlens"]),
              scale=fx["scale"], pool=np.array(fx["pool"]), state_indices=np.array(fx["state_indices"]),
              l2_eps=0.0)
    kw.update(over)
    return kda_front.kda_decode_front(**kw)


def test_hand_worked_example():
    with open(GOLDEN) as f:
        fx = json.load(f)
    r = _golden_front(fx)
    np.testing.assert_allclose(r["q"], fx["expected_q"], rtol=1e-15)
    np.testing.assert_allclose(r["k"], fx["expected_k"], rtol=1e-15)
    np.testing.assert_allclose(r["v"], fx["expected_v"], rtol=1e-15)
    np.testing.assert_allclose(r["g"], fx["expected_g"], rtol=1e-15)
    np.testing.assert_array_equal(r["conv"][0], fx["expected_window"])
    np.testing.assert_allclose(r["final"][0], fx["expected_state"], rtol=1e-12)
    np.testing.assert_allclose(r["o"], fx["expected_o"], rtol=1e-12)
    re = _golden_front(fx, norm_weight=np.array(fx["norm_weight"]), norm_gate=np.array(fx["norm_gate"]),
                       norm_eps=0.0)
    np.testing.assert_allclose(re["o"], fx["expected_o_epilogue"], rtol=1e-12)


def test_negative_controls_fail_the_example(monkeypatch):
    """Mistakes planted in the oracle move the hand-worked example's outputs past 1e-3: no
    convolution (current input only), no q/k normalisation, the gate without its softplus, and a
    decay of exp(+g)."""
    with open(GOLDEN) as f:
        fx = json.load(f)
    want = np.array(fx["expected_o"])
    assert np.allclose(_golden_front(fx)["o"], want, rtol=1e-12)
    # no convolution: identity taps on the current input only
    r = _golden_front(fx, conv_weight=np.array([[0.0, 1.0]] * 6))
    assert not np.allclose(r["o"], want, rtol=1e-3)
    with monkeypatch.context() as m:
        m.setattr(kda_front, "l2norm", lambda x, eps: np.asarray(x, dtype=np.float64))
        assert not np.allclose(_golden_front(fx)["o"], want, rtol=1e-3)
    with monkeypatch.context() as m:
        m.setattr(kda_front, "softplus", lambda x: np.asarray(x, dtype=np.float64))
        assert not np.allclose(_golden_front(fx)["o"], want, rtol=1e-3)
    with monkeypatch.context() as m:
        real = kda_front.kda_gate
        m.setattr(kda_front, "kda_gate", lambda *args: -real(*args))
        r = _golden_front(fx)
        assert not np.allclose(r["o"], want, rtol=1e-3)
