"""Context-parallel chunked path: one long sequence with few heads is cut into segments that run
in parallel (segment offsets, segment linear maps, a scan, then every segment from its true start
state).  Checked against the fp64 token oracle, with and without an initial state, for both gate
kinds and for fp32 operands."""
import numpy as np
import pytest
import torch

import oracle
from _cmp import TOL, max_rel_l2_states, max_rel_l2_tokens
from _dev import f64, oracle_inputs, problem_to_dev, to_dev
from gated_delta_rule_63_amd import gdr, inputs

pytestmark = pytest.mark.gpu


def _run_and_check(p, h0=True, with_cu=True):
    d = problem_to_dev(p)
    need = gdr.gdr_chunk_workspace_size(d["q"], d["v"], d["g"], 1)
    assert need > 0, "this shape is expected to take the segmented path"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, ht = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"] if with_cu else None, p.scale,
                              d.get("h0") if h0 else None, workspace=ws)
    torch.cuda.synchronize()
    q, k, v, g, beta = oracle_inputs(p)
    o_ref, f_ref, _ = oracle.recurrent(q, k, v, g, beta, p.cu_seqlens, p.scale, p.initial_state if h0 else None)
    oh, hh = f64(o), f64(ht)
    assert np.all(np.isfinite(oh)) and np.all(np.isfinite(hh))
    eo = max_rel_l2_tokens(oh, o_ref, p.cu_seqlens)
    es = max_rel_l2_states(hh, f_ref)
    tol = TOL[p.io_dtype]
    assert eo <= tol and es <= tol, f"o relL2 {eo}, state relL2 {es}"
    return o, ht


@pytest.mark.parametrize("h0,with_cu", [(True, True), (False, False)])
def test_gdn_bf16_single_long_sequence(h0, with_cu):
    p = inputs.dense_problem(81, [64 * 100 + 17], HK=1, HV=2, K=128, V=128, io_dtype="bf16",
                             g_range=(-0.5, 0.0))
    _run_and_check(p, h0=h0, with_cu=with_cu)


def test_gdn_bf16_adversarial_decay_gqa():
    p = inputs.dense_problem(82, [64 * 72 + 63], HK=1, HV=4, K=128, V=128, io_dtype="bf16", g_range=(-2.0, 0.0),
                             g_endpoints=0.25)
    _run_and_check(p)


def test_kda_bf16_single_long_sequence():
    p = inputs.dense_problem(83, [64 * 90 + 5], HK=2, HV=2, K=128, V=128, io_dtype="bf16", g_range=(-2.0, 0.0),
                             g_endpoints=0.25, per_k_gate=True, beta_mode="mixed", with_initial_state=False)
    _run_and_check(p, h0=False)


def test_fp32_k64_single_long_sequence():
    p = inputs.dense_problem(84, [64 * 60 + 5], HK=1, HV=2, K=64, V=64, io_dtype="f32", g_range=(-0.5, 0.0))
    _run_and_check(p)


def test_segmented_path_is_deterministic():
    p = inputs.dense_problem(85, [64 * 50 + 9], HK=1, HV=2, K=128, V=128, io_dtype="bf16")
    o1, h1 = _run_and_check(p)
    o2, h2 = _run_and_check(p)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_segmented_path_graph_capture_replay_equals_eager():
    """The segmented route (setup, three chunk runs, scan, copy) is capturable: it allocates
    nothing and records no memset; every replay equals the eager result bit for bit."""
    p = inputs.dense_problem(86, [64 * 50 + 3], HK=1, HV=2, K=128, V=128, io_dtype="bf16")
    d = problem_to_dev(p)
    need = gdr.gdr_chunk_workspace_size(d["q"], d["v"], d["g"], 1)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.zeros((p.T, p.HV, p.V), dtype=torch.bfloat16, device="cuda")
    ht = torch.zeros((1, p.HV, p.V, p.K), dtype=torch.float32, device="cuda")

    def call():
        gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale, d["h0"], o=o,
                          final_state=ht, workspace=ws)

    call()
    torch.cuda.synchronize()
    o_ref, ht_ref = o.clone(), ht.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(3):
        o.zero_()
        ht.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)


def test_gating_prepass_graph_capture_replay_equals_eager():
    r = inputs.raw_gating(87, 300, 2, 8, 128)
    dq, dk, da, db, A_log, dt = (to_dev(x) for x in (r.q, r.k, r.a, r.b, r.A_log, r.dt_bias))
    qo, ko = torch.zeros_like(dq), torch.zeros_like(dk)
    g = torch.zeros((300, 8), dtype=torch.float32, device="cuda")
    beta = torch.zeros((300, 8), dtype=torch.bfloat16, device="cuda")

    def call():
        gdr.gdr_gating_prepass(dq, dk, da, db, A_log, dt, q_out=qo, k_out=ko, g_out=g, beta_out=beta)

    call()
    torch.cuda.synchronize()
    refs = [t.clone() for t in (qo, ko, g, beta)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(3):
        for t in (qo, ko, g, beta):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(t, r_) for t, r_ in zip((qo, ko, g, beta), refs))
