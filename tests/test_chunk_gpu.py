"""Chunked path (gdr_chunk_fwd: the fused kernel running the intra-chunk WY/UT transform, the
inter-chunk state pass and the chunk output per 64-token chunk) against the fp64 token oracle."""
import numpy as np
import pytest
import torch

import oracle
from _cmp import TOL, max_rel_l2_states, max_rel_l2_tokens
from _dev import f64, oracle_inputs, problem_to_dev
from gated_delta_rule_63_amd import gdr, inputs

pytestmark = pytest.mark.gpu


def _chunk(p, d=None, h0=True, workspace=None):
    d = d or problem_to_dev(p)
    o, ht = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale,
                              d.get("h0") if h0 else None, workspace=workspace)
    torch.cuda.synchronize()
    return o, ht


def _check(p, o, ht, h0=True):
    q, k, v, g, beta = oracle_inputs(p)
    o_ref, f_ref, _ = oracle.recurrent(q, k, v, g, beta, p.cu_seqlens, p.scale, p.initial_state if h0 else None)
    oh, hh = f64(o), f64(ht)
    assert np.all(np.isfinite(oh)) and np.all(np.isfinite(hh))
    eo = max_rel_l2_tokens(oh, o_ref, p.cu_seqlens)
    es = max_rel_l2_states(hh, f_ref)
    tol = TOL[p.io_dtype]
    assert eo <= tol and es <= tol, f"o relL2 {eo}, state relL2 {es}"
    return eo, es


def test_tiny_fp32_one_chunk():
    p = inputs.tiny()
    o, ht = _chunk(p, h0=False)
    _check(p, o, ht, h0=False)


@pytest.mark.parametrize("lengths", [[1], [65, 1], [65, 63], [1024], [1] * 32, [64], [1, 37, 63, 64, 65, 130, 200]])
def test_gdn_bf16_lengths(lengths):
    """Sequence-length cases with partial tails (1, 37, 63, 65) and exact chunk multiples."""
    p = inputs.dense_problem(41 + len(lengths), lengths, HK=4, HV=4, K=128, V=128, io_dtype="bf16")
    o, ht = _chunk(p)
    _check(p, o, ht)


@pytest.mark.parametrize("HK,HV,lengths", [(2, 4, [1, 63, 65, 2]), (1, 4, [4]), (2, 8, [65, 1, 129, 63])])
def test_gqa_packed(HK, HV, lengths):
    p = inputs.dense_problem(50 + HV, lengths, HK=HK, HV=HV, K=128, V=128, io_dtype="bf16")
    o, ht = _chunk(p)
    _check(p, o, ht)


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64)])
def test_head_dims_bf16(K, V):
    p = inputs.dense_problem(60 + K + V, [100, 37], HK=2, HV=2, K=K, V=V, io_dtype="bf16")
    o, ht = _chunk(p)
    _check(p, o, ht)


@pytest.mark.parametrize("V,lengths,h0", [(128, [70, 5, 64, 200], True), (64, [130, 1, 63], True),
                                           (128, [65, 0, 37], False)])
def test_fp32_k128(V, lengths, h0):
    """fp32 I/O at K = 128 (scalar gate): fp32 MFMA, K^T read from the row-major rows."""
    p = inputs.dense_problem(65 + V + len(lengths), lengths, HK=2, HV=4, K=128, V=V, io_dtype="f32",
                             g_range=(-0.5, 0.0), with_initial_state=h0)
    o, ht = _chunk(p, h0=h0)
    _check(p, o, ht, h0=h0)


@pytest.mark.parametrize("V,lengths", [(128, [300, 0, 65, 1]), (64, [129, 64])])
def test_fp32_per_key_gate_k128_runs_the_token_kernel(V, lengths):
    """fp32 I/O with the per-key-channel gate at K = 128 (no chunked kernel fits the LDS): the chunk
    entry points run the token-serial kernel, so they equal gdr_recurrent_fwd bitwise, need no
    workspace, and meet the fp32 tolerance against the oracle."""
    p = inputs.dense_problem(67 + V, lengths, HK=2, HV=4, K=128, V=V, io_dtype="f32", g_range=(-2.0, 0.0),
                             g_endpoints=0.25, per_k_gate=True, beta_mode="mixed")
    d = problem_to_dev(p)
    assert gdr.gdr_chunk_workspace_size(d["q"], d["v"], d["g"], p.N) == 0
    o, ht = _chunk(p, d)
    _check(p, o, ht)
    o_r, ht_r = gdr.gdr_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale, d["h0"])
    o_n, ht_n = gdr.gdr_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale, d["h0"],
                                          o=torch.empty_like(o), final_state=torch.empty_like(ht))
    torch.cuda.synchronize()
    assert torch.equal(o, o_r) and torch.equal(ht, ht_r)
    assert torch.equal(o_n, o_r) and torch.equal(ht_n, ht_r)


@pytest.mark.parametrize("seed,lengths,K,V,HK,HV,lo,beta", [
    (10777, [1, 177, 127], 128, 64, 2, 8, -0.5, "mixed"),
    (10455, [128, 2000, 129, 1023, 256, 129, 256, 64, 1, 1818, 1557, 400, 63, 1432], 64, 64, 2, 4, -0.05, "one")])
def test_per_key_gate_one_token_sequence_with_cancelling_q_dot_k(seed, lengths, K, V, HK, HV, lo, beta):
    """A one-token sequence's output is scale (q . k) beta v: when q . k nearly cancels, the bf16 rounding
    of the per-channel scaled operands alone gave per-slice errors up to 0.65; the diagonal of P is summed
    from the unscaled rows, and every slice meets the bf16 tolerance (cases found by a seeded sweep)."""
    p = inputs.dense_problem(seed, lengths, HK=HK, HV=HV, K=K, V=V, io_dtype="bf16", g_range=(lo, 0.0),
                             per_k_gate=True, beta_mode=beta, with_initial_state=False)
    o, ht = _chunk(p, h0=False)
    _check(p, o, ht, h0=False)


def test_fp32_k128_adversarial_decay():
    p = inputs.dense_problem(66, [200, 64, 65], HK=1, HV=2, K=128, V=128, io_dtype="f32", g_range=(-2.0, 0.0),
                             g_endpoints=0.25)
    o, ht = _chunk(p)
    _check(p, o, ht)


@pytest.mark.parametrize("V", [64, 128])
def test_fp32_k64(V):
    p = inputs.dense_problem(61 + V, [70, 5, 64], HK=1, HV=2, K=64, V=V, io_dtype="f32", g_range=(-0.5, 0.0))
    o, ht = _chunk(p)
    _check(p, o, ht)


def test_adversarial_scalar_decay_endpoints():
    """g in U[-2, 0] with 25% exactly 0 and 25% exactly -2: 64-token prefixes reach -128."""
    p = inputs.dense_problem(70, [200, 64, 65], HK=4, HV=4, K=128, V=128, io_dtype="bf16", g_range=(-2.0, 0.0),
                             g_endpoints=0.25)
    o, ht = _chunk(p)
    _check(p, o, ht)


def test_kda_mixed_gates_and_betas():
    p = inputs.dense_problem(71, [130, 37, 64], HK=2, HV=2, K=128, V=128, io_dtype="bf16", g_range=(-2.0, 0.0),
                             g_endpoints=0.25, per_k_gate=True, beta_mode="mixed")
    o, ht = _chunk(p)
    _check(p, o, ht)


def test_kda_exp_minus_prefix_overflow_case():
    """All gk = -2, beta = 1, T = 200: a factored exp(-prefix) would overflow from the 45th
    token of each chunk; the outputs must stay finite and match the oracle."""
    p = inputs.kda_overflow_case()
    o, ht = _chunk(p, h0=False)
    _check(p, o, ht, h0=False)


@pytest.mark.parametrize("lo,io,K", [(-20.0, "bf16", 128), (-6.0, "bf16", 128), (-20.0, "f32", 64)])
def test_kda_wide_decay_range(lo, io, K):
    """Per-channel decays whose range over a 16-row block exceeds e^64 on some channels (gk down to
    -20: up to 320 per block; -6: around the limit): those chunks evaluate their diagonal blocks
    element-wise, the others on MFMA; every chunk must match the oracle."""
    p = inputs.dense_problem(73 + int(-lo), [200, 65, 7], HK=2, HV=2, K=K, V=K, io_dtype=io, g_range=(lo, 0.0),
                             g_endpoints=0.1, per_k_gate=True, beta_mode="mixed")
    o, ht = _chunk(p)
    _check(p, o, ht)


def test_kda_fp32_k64():
    p = inputs.dense_problem(72, [90, 3], HK=1, HV=2, K=64, V=64, io_dtype="f32", g_range=(-1.0, 0.0),
                             per_k_gate=True)
    o, ht = _chunk(p)
    _check(p, o, ht)


def test_chunked_matches_recurrent_on_gpu_and_repeats_bitwise():
    p = inputs.dense_problem(73, [300, 17, 128], HK=4, HV=8, K=128, V=128, io_dtype="bf16")
    d = problem_to_dev(p)
    o1, h1 = _chunk(p, d)
    o2, h2 = _chunk(p, d)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    orr, hr = gdr.gdr_recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale, d["h0"])
    torch.cuda.synchronize()
    assert max_rel_l2_tokens(f64(o1), f64(orr), p.cu_seqlens) <= TOL["bf16"]
    assert max_rel_l2_states(f64(h1), f64(hr)) <= TOL["bf16"]


@pytest.mark.parametrize("row", ["64", "1024", "packed4096", "boundary_x8", "gva2", "gva4"])
def test_repeated_launches_stay_bitwise_identical(row):
    """Determinism under repetition, scaled down from the cuLA PR #113 stress (100,000 launches over
    six rows): 300 back-to-back launches of each row, every one bitwise equal to the first.  Rows: one
    64-token sequence, one of 1024, 4096 tokens packed into sequences of 7..694, [1, 63, 64, 65] x 8,
    and the GVA2 [1, 63, 65, 2] and GVA4 [65, 1, 129, 63] batches (16 key heads)."""
    rng = np.random.default_rng(91)
    if row == "packed4096":
        lengths, left = [], 4096
        while left > 0:
            n = min(left, int(rng.integers(7, 695)))
            lengths.append(n)
            left -= n
    else:
        lengths = {"64": [64], "1024": [1024], "boundary_x8": [1, 63, 64, 65] * 8, "gva2": [1, 63, 65, 2],
                   "gva4": [65, 1, 129, 63]}[row]
    HV = {"gva2": 32, "gva4": 64}.get(row, 16)
    p = inputs.dense_problem(92, lengths, HK=16, HV=HV, K=128, V=128, io_dtype="bf16")
    d = problem_to_dev(p)
    o_ref, h_ref = _chunk(p, d)
    o, h = torch.empty_like(o_ref), torch.empty_like(h_ref)
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(300):
        gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale, d["h0"], o=o, final_state=h)
        bad += (o.view(torch.int16) != o_ref.view(torch.int16)).any().long()
        bad += (h.view(torch.int32) != h_ref.view(torch.int32)).any().long()
    torch.cuda.synchronize()
    assert int(bad) == 0


def test_inputs_untouched_flow_and_per_key_gate():
    """q, k, v, g, beta, cu_seqlens and the initial state are byte-identical after a call, on the flow
    kernel (scalar gate, bf16, K = V = 128) and on the per-key-channel kernel."""
    for per_k, seed in ((False, 75), (True, 76)):
        p = inputs.dense_problem(seed, [150, 64, 3], HK=2, HV=4, K=128, V=128, io_dtype="bf16", per_k_gate=per_k)
        d = problem_to_dev(p)
        snap = {k: v.clone() for k, v in d.items()}
        _chunk(p, d)
        for k in d:
            assert torch.equal(d[k], snap[k]), (per_k, k)


def test_empty_sequences_and_no_initial_state():
    p = inputs.dense_problem(74, [0, 70, 0, 5], HK=2, HV=2, K=128, V=128, io_dtype="bf16")
    o, ht = _chunk(p)
    _check(p, o, ht)
    np.testing.assert_array_equal(f64(ht)[0], p.initial_state[0])
    o, ht = _chunk(p, h0=False)
    _check(p, o, ht, h0=False)


def test_chunk_runs_without_workspace():
    p = inputs.dense_problem(76, [100, 3], HK=2, HV=2, K=128, V=128, io_dtype="bf16")
    d = problem_to_dev(p)
    assert gdr.gdr_chunk_workspace_size(d["q"], d["v"], d["g"], p.N) == 0
    o1, h1 = _chunk(p, d)
    o2, h2 = _chunk(p, d, workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    _check(p, o1, h1)


def test_outputs_stay_in_their_rows_and_final_state_in_place():
    """Every token row of o is written, nothing past the last row is, and the final state can overwrite
    the initial state in place (lengths cover both buffer parities of the chunk loop and short tails)."""
    lengths = [1, 63, 64, 65, 128, 129, 200]
    p = inputs.dense_problem(77, lengths, HK=2, HV=4, K=128, V=128, io_dtype="bf16")
    d = problem_to_dev(p)
    guard = 64
    sentinel = 0x7FC1  # a bf16 NaN pattern
    o_big = torch.full((p.T + guard, p.HV, p.V), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    o = o_big[: p.T]
    state = d["h0"].clone()  # initial state in, final state out, same memory
    gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale, state, o=o, final_state=state)
    torch.cuda.synchronize()
    tail = o_big[p.T:].view(torch.int16)
    assert bool((tail == sentinel).all()), "rows past the end were written"
    _check(p, o, state)


def test_varlen_prefill_graph_capture_replay_equals_eager():
    """A varlen prefill call (several sequences, the pipelined kernel) is capturable: it allocates
    nothing and records no memset; every replay, with eager work between replays, equals the eager
    result bit for bit."""
    p = inputs.dense_problem(78, [65, 130, 1, 64], HK=2, HV=4, K=128, V=128, io_dtype="bf16")
    d = problem_to_dev(p)
    o = torch.zeros((p.T, p.HV, p.V), dtype=torch.bfloat16, device="cuda")
    ht = torch.zeros((p.N, p.HV, p.V, p.K), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")

    def call():
        gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale, d["h0"], o=o,
                          final_state=ht, workspace=ws)

    call()
    torch.cuda.synchronize()
    o_ref, ht_ref = o.clone(), ht.clone()
    _check(p, o_ref, ht_ref)
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
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)


@pytest.mark.parametrize("seed", range(200, 210))
def test_random_shapes_bf16_k128(seed):
    """Seeded random shapes through the bf16, scalar-gate, K = V = 128 path (the pipelined kernel):
    1-12 sequences of 0-300 tokens, GQA ratios 1, 2 and 4, decay ranges up to [-2, 0], with and
    without an initial state."""
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 13))
    lengths = [int(x) for x in rng.integers(0, 301, size=N)]
    if sum(lengths) == 0:
        lengths[0] = 1  # empty batches are covered on their own
    HK = int(rng.choice([1, 2, 4]))
    HV = HK * int(rng.choice([1, 2, 4]))
    lo = float(rng.choice([-0.1, -0.5, -2.0]))
    p = inputs.dense_problem(seed, lengths, HK=HK, HV=HV, K=128, V=128, io_dtype="bf16", g_range=(lo, 0.0))
    with_h0 = bool(rng.integers(0, 2))
    o, ht = _chunk(p, h0=with_h0)
    _check(p, o, ht, h0=with_h0)


def _full_check(p, o, ht, h0=True):
    """Every (sequence, head) slice of o and of the final state against the oracle, at full size;
    every output value finite."""
    oh, hh = f64(o), f64(ht)
    assert np.all(np.isfinite(oh)) and np.all(np.isfinite(hh))
    q, k, v, g, beta = oracle_inputs(p)
    o_ref, f_ref, _ = oracle.recurrent(q, k, v, g, beta, p.cu_seqlens, p.scale, p.initial_state if h0 else None)
    del q, k, v, g, beta
    eo = max_rel_l2_tokens(oh, o_ref, p.cu_seqlens)
    es = max_rel_l2_states(hh, f_ref)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], f"o relL2 {eo}, state relL2 {es}"


def test_prefill_full_size_every_head():
    """8 ragged sequences, 32768 tokens, 32 heads, bf16, fp32 initial state: all 256 (sequence, head)
    slices of o and the final state against the oracle."""
    p = inputs.prefill()
    assert p.T == 32768 and 64 in p.lengths and 65 in p.lengths
    o, ht = _chunk(p)
    _full_check(p, o, ht)


def test_prefill_adversarial_full_size_every_head():
    """As the prefill workload with g in U[-2, 0] and 25% / 25% endpoints {0, -2}: every slice."""
    p = inputs.prefill(adversarial=True)
    o, ht = _chunk(p)
    _full_check(p, o, ht)


def test_kda_full_size_every_head():
    """One sequence of 65573 tokens (1025 chunks, last one 37 long), 16 heads, per-K gate: every head."""
    p = inputs.kda()
    o, ht = _chunk(p, h0=False)
    _full_check(p, o, ht, h0=False)
