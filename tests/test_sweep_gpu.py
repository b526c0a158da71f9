"""Seeded random sweep over the configuration space of every entry point, each case against the
fp64 oracle: the chunk entry (both I/O dtypes, K and V in {64, 128}, both gates, GQA ratios, decay
ranges up to [-2, 0] with endpoint mass, beta mixes, with and without an initial state or a
workspace, lengths on and around the chunk boundaries, empty sequences), paged decode and verify
(q_len 1..12, ragged, padded slots, commit or not, per-token states in either dtype), the gated
decode (l2norm on or off, doubled beta) and the fused KDA decode front (widths 1-4, ranks 8-264,
bias and epilogue on or off).  Tolerances and slot rules are those of the per-entry tests."""
import numpy as np
import pytest
import torch

import oracle
import test_gating_gpu as TG
import test_kda_front_gpu as TK
import test_paged_gpu as TP
from _cmp import TOL, max_rel_l2_states, max_rel_l2_tokens
from _dev import f64, oracle_inputs, problem_to_dev
from gated_delta_rule_63_amd import gdr, inputs

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 2, 37, 63, 64, 65, 127, 128, 129, 191, 200, 256, 300, 400]


@pytest.mark.parametrize("seed", range(5000, 5040))
def test_chunk_sweep(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 9))
    lengths = [int(rng.choice(LENGTHS)) if rng.uniform() < 0.6 else int(rng.integers(0, 450)) for _ in range(N)]
    if sum(lengths) == 0:
        lengths[0] = 1
    io = str(rng.choice(["bf16", "f32"]))
    K, V = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    HK = int(rng.choice([1, 2, 4]))
    HV = HK * int(rng.choice([1, 2, 4]))
    h0 = bool(rng.integers(0, 2))
    p = inputs.dense_problem(seed, lengths, HK=HK, HV=HV, K=K, V=V, io_dtype=io,
                             g_range=(float(rng.choice([-0.05, -0.5, -2.0])), 0.0),
                             g_endpoints=float(rng.choice([0.0, 0.0, 0.25])), per_k_gate=bool(rng.uniform() < 0.35),
                             beta_mode=str(rng.choice(["sigmoid", "sigmoid", "mixed", "one"])), with_initial_state=h0)
    d = problem_to_dev(p)
    ws = None
    if rng.integers(0, 2):
        ws = torch.empty(max(256, gdr.gdr_chunk_workspace_size(d["q"], d["v"], d["g"], p.N)), dtype=torch.uint8,
                         device="cuda")
    o, ht = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale,
                              d.get("h0") if h0 else None, workspace=ws)
    torch.cuda.synchronize()
    q, k, v, g, beta = oracle_inputs(p)
    o_ref, f_ref, _ = oracle.recurrent(q, k, v, g, beta, p.cu_seqlens, p.scale, p.initial_state if h0 else None)
    oh, hh = f64(o), f64(ht)
    assert np.all(np.isfinite(oh)) and np.all(np.isfinite(hh))
    eo, es = max_rel_l2_tokens(oh, o_ref, p.cu_seqlens), max_rel_l2_states(hh, f_ref)
    assert eo <= TOL[io] and es <= TOL[io], f"o relL2 {eo}, state relL2 {es}"


def _paged_case(rng, seed):
    B, ql = int(rng.integers(1, 41)), int(rng.integers(1, 13))
    K, V = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    HK = int(rng.choice([1, 2, 4]))
    HV = HK * int(rng.choice([1, 2, 4]))
    ib = str(rng.choice(["none", "bf16", "f32"]))
    commit = bool(rng.integers(0, 2))
    p = inputs.paged_problem(seed, B=B, q_len=ql, HK=HK, HV=HV, K=K, V=V, num_slots=B + 8,
                             pool_dtype=str(rng.choice(["f32", "bf16"])), io_dtype=str(rng.choice(["bf16", "f32"])),
                             pad_count=int(rng.integers(0, B // 3 + 1)), commit=commit,
                             ragged=bool(rng.integers(0, 2)), inter_dtype=None if ib == "none" else ib, cache_steps=ql)
    ibt = None if ib == "none" else (torch.bfloat16 if ib == "bf16" else torch.float32)
    return p, ibt, commit


def _check_paged(p, before, o, pool, ib, ibt, ref, commit):
    TP._check_o(p, o, ref)
    TP._check_pool(p, before, pool, ref, committed=commit)
    if ibt is not None:
        TP._check_ibuf(p, ib, ref)


@pytest.mark.parametrize("seed", range(6000, 6030))
def test_paged_sweep(seed):
    rng = np.random.default_rng(seed)
    p, ibt, commit = _paged_case(rng, seed)
    if rng.uniform() < 0.3:  # per-key-channel gate
        p = inputs.paged_problem(seed, B=p.N, q_len=p.max_q_len, HK=p.HK, HV=p.HV, K=p.K, V=p.V, num_slots=p.N + 8,
                                 pool_dtype=p.pool_dtype, io_dtype=p.io_dtype, pad_count=int((p.state_indices < 0).sum()),
                                 commit=commit, per_k_gate=True,
                                 inter_dtype=None if ibt is None else ("bf16" if ibt == torch.bfloat16 else "f32"),
                                 cache_steps=p.max_q_len)
    before = p.pool.copy()
    o, pool, ib = TP._run(p, with_ibuf=ibt)
    q, k, v, g, beta = oracle_inputs(p)
    ref = oracle.decode_paged(q, k, v, g, beta, p.cu_seqlens, p.scale, inputs.widen(p.pool), p.state_indices,
                              want_states=ibt is not None)
    _check_paged(p, before, o, pool, ib, ibt, ref, commit)


@pytest.mark.parametrize("seed", range(7000, 7030))
def test_gated_sweep(seed):
    rng = np.random.default_rng(seed)
    p, ibt, commit = _paged_case(rng, seed)
    r = inputs.raw_gating(seed + 7, p.T, p.HK, p.HV, p.K, io_dtype=p.io_dtype,
                          allow_neg_eigval=bool(rng.integers(0, 2)), qk_l2norm=bool(rng.uniform() < 0.8))
    before = p.pool.copy()
    o, pool, ib = TG._run_gated(p, r, with_ibuf=ibt)
    ref = TG._ref(p, r, want_states=ibt is not None)
    _check_paged(p, before, o, pool, ib, ibt, ref, commit)


@pytest.mark.parametrize("seed", range(8000, 8030))
def test_kda_front_sweep(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 17))
    commit = bool(rng.integers(0, 2))
    p = inputs.kda_front_problem(seed, B=B, q_len=int(rng.integers(1, 13)), H=int(rng.integers(1, 5)),
                                 K=int(rng.choice([64, 128])), V=int(rng.choice([64, 128])),
                                 R=int(rng.choice([8, 16, 40, 128, 200, 264])), W=int(rng.integers(1, 5)),
                                 io_dtype=str(rng.choice(["bf16", "f32"])), pool_dtype=str(rng.choice(["f32", "bf16"])),
                                 pad_count=int(rng.integers(0, B // 3 + 1)), ragged=bool(rng.integers(0, 2)),
                                 with_bias=bool(rng.integers(0, 2)), with_epilogue=bool(rng.integers(0, 2)))
    o, pool, conv = TK._run(p, commit=commit)
    TK._check(p, o, pool, conv, commit=commit)
