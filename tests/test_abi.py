"""CPU-side checks of the C ABI: the library loads, exports every entry point the header
declares, and rejects bad metadata on the host before touching the device."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_63_amd import gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "gdr.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"GDR_API\s+[\w\s\*]+?\b(gdr_\w+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    syms = _declared_symbols()
    for name in ("gdr_recurrent_fwd", "gdr_chunk_fwd", "gdr_decode_paged", "gdr_chunk_workspace_size",
                 "gdr_status_string", "gdr_gating_prepass", "gdr_decode_paged_gated"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    L = gdr.lib()
    for name in _declared_symbols():
        assert hasattr(L, name), name


def test_status_strings():
    assert gdr.gdr_status_string(0) == "GDR_SUCCESS"
    assert gdr.gdr_status_string(1) == "GDR_ERROR_INVALID_VALUE"
    assert gdr.gdr_status_string(2) == "GDR_ERROR_NOT_SUPPORTED"
    assert gdr.gdr_status_string(3) == "GDR_ERROR_LAUNCH_FAILED"
    assert gdr.gdr_status_string(4) == "GDR_ERROR_SCRATCH_LIMIT"
    assert gdr.gdr_status_string(99) == "GDR_ERROR_UNKNOWN"


def _p(T=8, N=1, HK=1, HV=2, K=128, V=128, gate=0, io=1):
    return gdr.Problem(T, N, HK, HV, K, V, 0.1, gate, io)


DUMMY = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails before any launch


def _rec(p, **kw):
    args = dict(q=DUMMY, k=DUMMY, v=DUMMY, g=DUMMY, beta=DUMMY, cu=None, h0=None, o=DUMMY, ht=None)
    args.update(kw)
    return gdr.lib().gdr_recurrent_fwd(ctypes.byref(p) if p is not None else None, args["q"], args["k"], args["v"],
                                       args["g"], args["beta"], args["cu"], args["h0"], args["o"], args["ht"], None)


@pytest.mark.parametrize("field,value,expect", [
    ("num_v_heads", 3, 1),       # HV % HK != 0 with HK = 2 below
    ("head_dim_k", 96, 2),
    ("head_dim_v", 32, 2),
    ("head_dim_k", 0, 1),
    ("gate", 7, 1),
    ("io_dtype", 5, 1),
    ("total_tokens", -1, 1),
    ("num_seqs", -1, 1),
])
def test_recurrent_rejects_bad_metadata(field, value, expect):
    p = _p(HK=2, HV=4)
    setattr(p, field, value)
    assert _rec(p) == expect


def test_recurrent_rejects_null_pointers():
    assert _rec(None) == 1
    assert _rec(_p(), q=None) == 1
    assert _rec(_p(), o=None) == 1
    assert _rec(_p(N=2)) == 1  # cu_seqlens required for N > 1


def test_empty_problems_succeed_without_touching_the_device():
    assert _rec(_p(T=0, N=0), q=None, k=None, v=None, g=None, beta=None, o=None) == 0
    assert _rec(_p(T=0, N=3), q=None, k=None, v=None, g=None, beta=None, o=None, cu=DUMMY) == 0


def _dec(p, max_q_len=1, **kw):
    a = dict(cu=None, pool=DUMMY, pool_dt=0, slots=4, idx=DUMMY, commit=1, ib=None, ib_dt=1, ncs=0, steps=0,
             ibidx=None)
    a.update(kw)
    return gdr.lib().gdr_decode_paged(ctypes.byref(p), max_q_len, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, a["cu"],
                                      a["pool"], a["pool_dt"], a["slots"], a["idx"], a["commit"], a["ib"],
                                      a["ib_dt"], a["ncs"], a["steps"], a["ibidx"], DUMMY, None)


def test_decode_rejects_bad_metadata():
    assert _dec(_p(T=4, N=4), max_q_len=0) == 1
    assert _dec(_p(T=4, N=4), max_q_len=13) == 1
    assert _dec(_p(T=5, N=4)) == 1                       # no cu_seqlens but T != N
    assert _dec(_p(T=30, N=2), max_q_len=12, cu=DUMMY) == 1  # T > N * max_q_len
    assert _dec(_p(T=4, N=4), pool=None) == 1
    assert _dec(_p(T=4, N=4), idx=None) == 1
    assert _dec(_p(T=4, N=4), slots=0) == 1
    assert _dec(_p(T=4, N=4), pool_dt=9) == 1
    assert _dec(_p(T=4, N=4), commit=2) == 1
    # intermediate buffer: indices, cache slots and cache_steps >= max_q_len are required
    assert _dec(_p(T=8, N=4), max_q_len=2, cu=DUMMY, ib=DUMMY, ncs=5, steps=2) == 1
    assert _dec(_p(T=8, N=4), max_q_len=2, cu=DUMMY, ib=DUMMY, ibidx=DUMMY, ncs=5, steps=1) == 1
    assert _dec(_p(T=8, N=4), max_q_len=2, cu=DUMMY, ib=DUMMY, ibidx=DUMMY, ncs=0, steps=2) == 1
    assert _dec(_p(T=0, N=4), cu=DUMMY) == 0  # nothing to do


def test_chunk_workspace_and_rejections():
    L = gdr.lib()
    p = _p(T=1000, N=3, HV=4)
    need = L.gdr_chunk_workspace_size(ctypes.byref(p), 64)
    assert need == 0  # every intermediate stays on chip
    assert L.gdr_chunk_workspace_size(ctypes.byref(p), 32) == 0
    bad = _p(K=96)
    assert L.gdr_chunk_workspace_size(ctypes.byref(bad), 64) == 0

    def call(p, cs=64, ws=DUMMY, nbytes=need, cu=DUMMY):
        return L.gdr_chunk_fwd(ctypes.byref(p), cs, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, cu, None, DUMMY, None,
                               ws, nbytes, None)
    assert call(p, cs=32) == 1
    assert call(p, ws=ctypes.c_void_p(0x1010)) == 1    # not 256-byte aligned
    assert call(p, cu=None) == 1                        # N > 1 needs cu_seqlens
    assert call(_p(K=96)) == 2
    assert call(_p(K=128, io=0, gate=1)) == 2           # fp32 with the per-channel gate needs K = 64


def test_chunk_noalloc_rejects_bad_metadata_before_the_device():
    L = gdr.lib()

    def call(p, cs=64, cu=DUMMY, o=DUMMY):
        return L.gdr_chunk_fwd_noalloc(ctypes.byref(p), cs, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, cu, None, o, None, None)
    p = _p(T=1000, N=3, HV=4)
    assert call(p, cs=32) == 1
    assert call(p, cu=None) == 1                        # N > 1 needs cu_seqlens
    assert call(p, o=None) == 1
    assert call(_p(K=96)) == 2
    assert call(_p(K=128, io=0, gate=1)) == 2
    assert call(_p(T=0, N=0), cu=None) == 0             # nothing to do, no device needed
    assert L.gdr_chunk_fwd_noalloc(None, 64, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY, None, None) == 1


@pytest.mark.parametrize("T,N,HV,K,V,io", [(65573, 1, 16, 128, 128, 1), (1 << 22, 1, 1, 128, 128, 1),
                                          (1 << 22, 1, 2, 128, 128, 1), (1 << 22, 1, 3, 128, 128, 1),
                                          (1 << 20, 1, 1, 64, 64, 0), (1 << 20, 1, 1, 128, 64, 1)])
def test_noalloc_scratch_covers_the_segmented_route(T, N, HV, K, V, io):
    """The fixed scratch of the no-alloc entry covers the workspace the segmented route plans for
    long sequences (its largest is one round of 256 segment-heads of 64 KiB states)."""
    p = gdr.Problem(T, N, 1, HV, K, V, 0.1, 0, io)
    need = gdr.lib().gdr_chunk_workspace_size(ctypes.byref(p), 64)
    assert 0 < need <= gdr.GDR_NOALLOC_SCRATCH_BYTES


def _gating(**kw):
    f = dict(a=0x1000, b=0x1000, A_log=0x1000, dt_bias=0x1000, l2norm_eps=1e-6, qk_l2norm=1, allow_neg_eigval=0)
    f.update(kw)
    return gdr.Gating(f["a"], f["b"], f["A_log"], f["dt_bias"], f["l2norm_eps"], f["qk_l2norm"],
                      f["allow_neg_eigval"])


def _pre(p, gt, q=DUMMY, k=DUMMY, qo=DUMMY, ko=DUMMY, g=DUMMY, b=DUMMY):
    return gdr.lib().gdr_gating_prepass(ctypes.byref(p), q, k, ctypes.byref(gt) if gt is not None else None,
                                        qo, ko, g, b, None)


def _decg(p, gt, max_q_len=1, **kw):
    a = dict(cu=None, pool=DUMMY, pool_dt=0, slots=4, idx=DUMMY, commit=1, ib=None, ib_dt=1, ncs=0, steps=0,
             ibidx=None, q=DUMMY)
    a.update(kw)
    return gdr.lib().gdr_decode_paged_gated(ctypes.byref(p), max_q_len, a["q"], DUMMY, DUMMY,
                                            ctypes.byref(gt) if gt is not None else None, a["cu"], a["pool"],
                                            a["pool_dt"], a["slots"], a["idx"], a["commit"], a["ib"], a["ib_dt"],
                                            a["ncs"], a["steps"], a["ibidx"], DUMMY, None)


def test_gated_entry_points_reject_bad_metadata():
    p = _p(T=4, N=4)
    for call in (lambda gt, **kw: _pre(p, gt, **kw), lambda gt, **kw: _decg(p, gt, **kw)):
        assert call(None) == 1
        assert call(_gating(qk_l2norm=2)) == 1
        assert call(_gating(allow_neg_eigval=-1)) == 1
        assert call(_gating(l2norm_eps=-1e-6)) == 1
        assert call(_gating(l2norm_eps=float("nan"))) == 1
        assert call(_gating(l2norm_eps=float("inf"))) == 1
        assert call(_gating(a=None)) == 1
        assert call(_gating(dt_bias=None)) == 1
    # the gating front defines a scalar decay only
    assert _pre(_p(T=4, N=4, gate=1), _gating()) == 2
    assert _decg(_p(T=4, N=4, gate=1), _gating()) == 2
    # pre-pass outputs; q/k outputs only matter when normalising
    assert _pre(p, _gating(), g=None) == 1
    assert _pre(p, _gating(), b=None) == 1
    assert _pre(p, _gating(), qo=None) == 1
    # decode checks apply to the gated variant as well
    assert _decg(p, _gating(), max_q_len=13) == 1
    assert _decg(p, _gating(), q=None) == 1
    assert _decg(_p(T=5, N=4), _gating()) == 1


def test_gated_entry_points_accept_empty_batches_without_the_device():
    assert _pre(_p(T=0, N=1), _gating(a=None, b=None, A_log=None, dt_bias=None), q=None, k=None, qo=None, ko=None,
                g=None, b=None) == 0
    assert _decg(_p(T=0, N=4), _gating(), cu=DUMMY) == 0


def _cp_size(T, N, HV, K=128, V=128, io=1):
    p = gdr.Problem(T, N, 1, HV, K, V, 0.1, 1, io)
    return gdr.lib().gdr_chunk_workspace_size(ctypes.byref(p), 64)


def _cp_expected(T, N, HV, K, V, io_bytes):
    """Workspace of the segmented path, written out from its definition: segments target one
    workgroup per (segment, head) on 256 CUs (at least 4 segments per sequence in that round), with
    at least 8 chunks each, and at least 4 segments per sequence on average; the workspace holds
    the segment table, the per-sequence first-segment indices, and P offsets [HV, V, K], P maps
    [HV, K, K] and P start states [HV, V, K], where P = floor(T / segment) + N bounds the segment
    count for any lengths; each part rounded up to 256 bytes."""
    vt = V // 64 if io_bytes == 4 else 1
    per_seq = 256 // (N * HV * vt)
    if per_seq < 4:
        return 0
    nchunks = (T + 63) // 64
    seg = 64 * max(8, -(-nchunks // (per_seq * N)))
    if T // seg // N < 4:
        return 0
    P = T // seg + N
    up = lambda x: -(-x // 256) * 256
    return (up(4 * (P + 1)) + up(4 * (N + 1)) + up(4 * P * HV * V * K) + up(4 * P * HV * K * K)
            + up(4 * P * HV * V * K))


def test_segment_bound_covers_every_length_split():
    """P = floor(T / seg) + N is at least sum_n max(1, ceil(len_n / seg)) for any lengths summing to T
    (brute force over small cases, empty sequences included)."""
    import itertools
    for seg in (3, 4, 7):
        for N in (1, 2, 3):
            for lens in itertools.product(range(0, 13), repeat=N):
                T = sum(lens)
                need = sum(max(1, -(-x // seg)) for x in lens)
                assert need <= T // seg + N, (seg, lens)


@pytest.mark.parametrize("T,N,HV,K,V,io", [(65573, 1, 16, 128, 128, 1), (6417, 1, 2, 128, 128, 1),
                                          (3845, 1, 2, 64, 64, 0), (65573, 2, 16, 128, 128, 1),
                                          (2000, 1, 16, 128, 128, 1), (64, 1, 2, 64, 64, 0),
                                          (32768, 1, 32, 128, 128, 1), (65573, 1, 64, 128, 128, 1),
                                          (65536, 4, 16, 128, 128, 1), (32768, 8, 32, 128, 128, 1),
                                          (9000, 3, 2, 128, 128, 1), (9000, 3, 2, 64, 128, 0),
                                          (1 << 20, 16, 4, 128, 128, 1)])
def test_segmented_workspace_size(T, N, HV, K, V, io):
    """Host-side planning of the context-parallel route: few long sequences with few heads take it;
    everything else needs no workspace."""
    got = _cp_size(T, N, HV, K, V, io)
    assert got == _cp_expected(T, N, HV, K, V, 4 if io == 0 else 2)
    if (T, N, HV) in ((65573, 1, 16), (65573, 2, 16), (65536, 4, 16)):
        assert got > 0  # the KDA stress shape and a few long GDN sequences are segmented
    if (T, N, HV) in ((32768, 8, 32), (2000, 1, 16)):
        assert got == 0  # the prefill workload (8 sequences, 32 heads) and short sequences are not


def test_fp32_per_key_gate_k128_needs_no_workspace():
    """fp32 I/O with the per-key-channel gate at K = 128 runs the token-serial kernel: no segmented
    route, so no workspace even for one long sequence with few heads; K = 64 keeps its route."""
    assert _cp_size(65573, 1, 16, 128, 128, io=0) == 0
    assert _cp_size(65573, 1, 16, 128, 64, io=0) == 0
    assert _cp_size(65573, 1, 16, 64, 64, io=0) == _cp_expected(65573, 1, 16, 64, 64, 4) > 0


def _kda_front(**kw):
    f = dict(conv_width=4, conv_weight=0x1000, conv_bias=None, conv_state=0x1000, gate_in=0x1000,
             gate_weight=0x1000, gate_rank=128, A_log=0x1000, dt_bias=0x1000, b=0x1000, l2norm_eps=1e-6,
             norm_weight=None, norm_gate=None, norm_eps=1e-6)
    f.update(kw)
    return gdr.KdaFront(f["conv_width"], f["conv_weight"], f["conv_bias"], f["conv_state"], f["gate_in"],
                        f["gate_weight"], f["gate_rank"], f["A_log"], f["dt_bias"], f["b"], f["l2norm_eps"],
                        f["norm_weight"], f["norm_gate"], f["norm_eps"])


def _kda(p, front, max_q_len=1, cu=None, pool=DUMMY, idx=DUMMY, commit=1, o=DUMMY, slots=8):
    return gdr.lib().gdr_kda_decode_fused(ctypes.byref(p), max_q_len, DUMMY, DUMMY, DUMMY,
                                          ctypes.byref(front) if front is not None else None, cu, pool, 0, slots, idx,
                                          commit, o, None)


def test_kda_front_rejects_bad_metadata_before_the_device():
    p = _p(T=4, N=4, HK=2, HV=2, gate=1)
    assert _kda(p, None) == 1
    assert _kda(p, _kda_front(conv_width=5)) == 1
    assert _kda(p, _kda_front(conv_width=0)) == 1
    assert _kda(p, _kda_front(conv_state=None)) == 1                 # W > 1 needs the windows
    assert _kda(p, _kda_front(gate_rank=12)) == 1                    # a multiple of 8
    assert _kda(p, _kda_front(gate_rank=0)) == 1
    assert _kda(p, _kda_front(l2norm_eps=-1.0)) == 1
    assert _kda(p, _kda_front(norm_weight=0x1000)) == 1              # the epilogue needs its gate
    assert _kda(p, _kda_front(b=None)) == 1
    assert _kda(p, _kda_front(), max_q_len=13) == 1
    assert _kda(p, _kda_front(), commit=2) == 1
    assert _kda(p, _kda_front(), pool=None) == 1
    assert _kda(p, _kda_front(), o=None) == 1
    assert _kda(_p(T=5, N=4, HK=2, HV=2, gate=1), _kda_front()) == 1  # T != N without cu_seqlens
    # the front is defined for the per-key-channel gate with one key head per value head
    assert _kda(_p(T=4, N=4, HK=2, HV=2, gate=0), _kda_front()) == 2
    assert _kda(_p(T=4, N=4, HK=1, HV=2, gate=1), _kda_front()) == 2
    # empty batch: nothing to do, no device needed
    assert _kda(_p(T=0, N=4, HK=2, HV=2, gate=1), _kda_front(), cu=DUMMY) == 0
