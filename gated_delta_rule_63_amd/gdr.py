"""Thin Python binding of libgdr.so (C ABI in include/gdr.h).

Argument marshalling only: every function checks that the torch tensors it is
given are contiguous device tensors of the documented shape and dtype, builds the
``gdr_problem`` struct, passes raw pointers and the current HIP stream, and raises
``GdrError`` on a non-success status.  All computation happens in the library's
HIP kernels.  If the library has not been built, loading it raises immediately.

Names follow the C entry points: ``gdr_recurrent_fwd``, ``gdr_chunk_fwd``,
``gdr_chunk_fwd_noalloc``, ``gdr_chunk_workspace_size``, ``gdr_decode_paged``,
``gdr_gating_prepass``, ``gdr_decode_paged_gated``, ``gdr_kda_decode_fused``, ``gdr_status_string``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_DEFAULT_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdr.so")
_LIB_PATH = _DEFAULT_LIB_PATH
_lib = None

GDR_SUCCESS, GDR_ERROR_INVALID_VALUE, GDR_ERROR_NOT_SUPPORTED, GDR_ERROR_LAUNCH_FAILED = 0, 1, 2, 3
GDR_ERROR_SCRATCH_LIMIT = 4
GDR_NOALLOC_SCRATCH_BYTES = 64 << 20
GDR_F32, GDR_BF16 = 0, 1
GDR_GATE_SCALAR, GDR_GATE_PER_K = 0, 1


class GdrError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {gdr_status_string(status)} ({status})")
        self.status = status


class Gating(ctypes.Structure):
    _fields_ = [
        ("a", ctypes.c_void_p),
        ("b", ctypes.c_void_p),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("l2norm_eps", ctypes.c_float),
        ("qk_l2norm", ctypes.c_int32),
        ("allow_neg_eigval", ctypes.c_int32),
    ]


class KdaFront(ctypes.Structure):
    _fields_ = [
        ("conv_width", ctypes.c_int32),
        ("conv_weight", ctypes.c_void_p),
        ("conv_bias", ctypes.c_void_p),
        ("conv_state", ctypes.c_void_p),
        ("gate_in", ctypes.c_void_p),
        ("gate_weight", ctypes.c_void_p),
        ("gate_rank", ctypes.c_int32),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("b", ctypes.c_void_p),
        ("l2norm_eps", ctypes.c_float),
        ("norm_weight", ctypes.c_void_p),
        ("norm_gate", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
    ]


class Problem(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32),
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("gate", ctypes.c_int),
        ("io_dtype", ctypes.c_int),
    ]


def library_path() -> str:
    return _LIB_PATH


def use_library(path: Optional[str] = None) -> None:
    """Bind to another build of the library from here on (the measurement build libgdr_stamps.so
    exports the same entry points, with the flow kernel's clock counters compiled in); None binds
    to libgdr.so again."""
    global _lib, _LIB_PATH
    _lib = None
    _LIB_PATH = path if path is not None else _DEFAULT_LIB_PATH


def lib():
    """Load libgdr.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m gated_delta_rule_63_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        P = ctypes.POINTER(Problem)
        L.gdr_status_string.restype = ctypes.c_char_p
        L.gdr_status_string.argtypes = [ctypes.c_int]
        L.gdr_recurrent_fwd.restype = ctypes.c_int
        L.gdr_recurrent_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdr_chunk_workspace_size.restype = ctypes.c_size_t
        L.gdr_chunk_workspace_size.argtypes = [P, i32]
        L.gdr_chunk_fwd.restype = ctypes.c_int
        L.gdr_chunk_fwd.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
        L.gdr_chunk_fwd_noalloc.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdr_decode_paged.restype = ctypes.c_int
        L.gdr_decode_paged.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, vp, i32,
                                       vp, ctypes.c_int, i32, i32, vp, vp, vp]
        G = ctypes.POINTER(Gating)
        L.gdr_gating_prepass.restype = ctypes.c_int
        L.gdr_gating_prepass.argtypes = [P, vp, vp, G, vp, vp, vp, vp, vp]
        L.gdr_decode_paged_gated.restype = ctypes.c_int
        L.gdr_decode_paged_gated.argtypes = [P, i32, vp, vp, vp, G, vp, vp, ctypes.c_int, i32, vp, i32,
                                             vp, ctypes.c_int, i32, i32, vp, vp, vp]
        L.gdr_kda_decode_fused.restype = ctypes.c_int
        L.gdr_kda_decode_fused.argtypes = [P, i32, vp, vp, vp, ctypes.POINTER(KdaFront), vp, vp, ctypes.c_int, i32, vp,
                                           i32, vp, vp]
        _lib = L
    return _lib


def gdr_status_string(status: int) -> str:
    return lib().gdr_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return GDR_F32
    if t == torch.bfloat16:
        return GDR_BF16
    raise TypeError(f"unsupported dtype {t}: use float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: Optional[torch.Tensor], name: str, shape=None, dtype=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (the C ABI sees no strides)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _problem(q, k, v, g, num_seqs: int, scale: Optional[float]) -> Problem:
    T, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    per_k = g.dim() == 3
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    return Problem(T, num_seqs, HK, HV, K, V, float(scale), GDR_GATE_PER_K if per_k else GDR_GATE_SCALAR,
                   _dtype_code(q.dtype))


def _check_tokens(q, k, v, g, beta):
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k are [T, HK, K] and v is [T, HV, V]")
    T, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    _check(q, "q")
    _check(k, "k", (T, HK, K), q.dtype)
    _check(v, "v", (T, HV, V), q.dtype)
    _check(beta, "beta", (T, HV), q.dtype)
    if g.dim() == 3:
        _check(g, "g", (T, HV, K), torch.float32)
    else:
        _check(g, "g", (T, HV), torch.float32)
    return T, HK, HV, K, V


def _num_seqs(cu_seqlens, default: int) -> int:
    if cu_seqlens is None:
        return default
    _check(cu_seqlens, "cu_seqlens", dtype=torch.int32)
    return cu_seqlens.shape[0] - 1


def _raise(status: int, where: str):
    if status != GDR_SUCCESS:
        raise GdrError(status, where)


# ---------------------------------------------------------------------------
def gdr_recurrent_fwd(q, k, v, g, beta, cu_seqlens=None, scale=None, initial_state=None, o=None,
                      final_state=None, output_final_state: bool = True, stream=None):
    """Token-by-token recurrence.  Returns (o, final_state or None)."""
    T, HK, HV, K, V = _check_tokens(q, k, v, g, beta)
    N = _num_seqs(cu_seqlens, 1)
    _check(initial_state, "initial_state", (N, HV, V, K), torch.float32, optional=True)
    if o is None:
        o = torch.empty((T, HV, V), dtype=q.dtype, device=q.device)
    _check(o, "o", (T, HV, V), q.dtype)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, HV, V, K), dtype=torch.float32, device=q.device)
    _check(final_state, "final_state", (N, HV, V, K), torch.float32, optional=True)
    p = _problem(q, k, v, g, N, scale)
    st = lib().gdr_recurrent_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(cu_seqlens), _ptr(initial_state), _ptr(o), _ptr(final_state), _stream(stream))
    _raise(st, "gdr_recurrent_fwd")
    return o, final_state


def gdr_chunk_workspace_size(q, v, g, num_seqs: int, chunk_size: int = 64) -> int:
    p = _problem(q, q, v, g, num_seqs, 1.0)
    return int(lib().gdr_chunk_workspace_size(ctypes.byref(p), int(chunk_size)))


def gdr_chunk_fwd(q, k, v, g, beta, cu_seqlens=None, scale=None, initial_state=None, o=None,
                  final_state=None, output_final_state: bool = True, workspace=None, chunk_size: int = 64,
                  stream=None, segmented: bool = True):
    """Chunked (64-token) forward.  Returns (o, final_state or None).  ``workspace`` is a
    uint8 device tensor of at least gdr_chunk_workspace_size bytes (allocated here if absent).
    ``segmented=False`` passes no workspace, which makes the library run every sequence in one
    pass even where it would cut few long sequences into segments."""
    T, HK, HV, K, V = _check_tokens(q, k, v, g, beta)
    N = _num_seqs(cu_seqlens, 1)
    _check(initial_state, "initial_state", (N, HV, V, K), torch.float32, optional=True)
    if o is None:
        o = torch.empty((T, HV, V), dtype=q.dtype, device=q.device)
    _check(o, "o", (T, HV, V), q.dtype)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, HV, V, K), dtype=torch.float32, device=q.device)
    _check(final_state, "final_state", (N, HV, V, K), torch.float32, optional=True)
    p = _problem(q, k, v, g, N, scale)
    need = int(lib().gdr_chunk_workspace_size(ctypes.byref(p), int(chunk_size)))
    if not segmented:
        workspace = None
    elif workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", dtype=torch.uint8, optional=True)
    st = lib().gdr_chunk_fwd(ctypes.byref(p), int(chunk_size), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(cu_seqlens), _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(workspace),
                             0 if workspace is None else workspace.numel(), _stream(stream))
    _raise(st, "gdr_chunk_fwd")
    return o, final_state


def gdr_chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens=None, scale=None, initial_state=None, o=None,
                          final_state=None, chunk_size: int = 64, stream=None):
    """gdr_chunk_fwd without a workspace argument: the library's fixed per-GPU scratch array
    (GDR_NOALLOC_SCRATCH_BYTES) stands in for it.  ``o`` must be given; the C call allocates
    nothing.  Calls that overlap on one GPU race on the scratch."""
    T, HK, HV, K, V = _check_tokens(q, k, v, g, beta)
    N = _num_seqs(cu_seqlens, 1)
    _check(initial_state, "initial_state", (N, HV, V, K), torch.float32, optional=True)
    _check(o, "o", (T, HV, V), q.dtype)
    _check(final_state, "final_state", (N, HV, V, K), torch.float32, optional=True)
    p = _problem(q, k, v, g, N, scale)
    st = lib().gdr_chunk_fwd_noalloc(ctypes.byref(p), int(chunk_size), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                     _ptr(beta), _ptr(cu_seqlens), _ptr(initial_state), _ptr(o), _ptr(final_state),
                                     _stream(stream))
    _raise(st, "gdr_chunk_fwd_noalloc")
    return o, final_state


def gdr_decode_paged(q, k, v, g, beta, pool, state_indices, cu_seqlens=None, max_q_len: int = 1,
                     commit: bool = True, inter_states=None, inter_state_indices=None, scale=None, o=None,
                     stream=None):
    """Paged decode / speculative verify.  pool [num_slots, HV, V, K] (float32 or bfloat16),
    state_indices int32 [N] (-1 = padded).  inter_states [num_cache_slots, cache_steps, HV, V, K]
    or None.  Returns o (rows of padded sequences are left as they were)."""
    T, HK, HV, K, V = _check_tokens(q, k, v, g, beta)
    _check(state_indices, "state_indices", dtype=torch.int32)
    N = state_indices.shape[0]
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)
    if pool.dim() != 4:
        raise ValueError("pool is [num_slots, HV, V, K]")
    _check(pool, "pool", (pool.shape[0], HV, V, K))
    pool_dt = _dtype_code(pool.dtype)
    ncs = steps = 0
    inter_dt = GDR_F32
    if inter_states is not None:
        if inter_states.dim() != 5:
            raise ValueError("inter_states is [num_cache_slots, cache_steps, HV, V, K]")
        ncs, steps = inter_states.shape[0], inter_states.shape[1]
        _check(inter_states, "inter_states", (ncs, steps, HV, V, K))
        inter_dt = _dtype_code(inter_states.dtype)
        _check(inter_state_indices, "inter_state_indices", (N,), torch.int32)
    if o is None:
        o = torch.empty((T, HV, V), dtype=q.dtype, device=q.device)
    _check(o, "o", (T, HV, V), q.dtype)
    p = _problem(q, k, v, g, N, scale)
    st = lib().gdr_decode_paged(ctypes.byref(p), int(max_q_len), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(cu_seqlens), _ptr(pool), pool_dt, pool.shape[0], _ptr(state_indices),
                                1 if commit else 0, _ptr(inter_states), inter_dt, ncs, steps,
                                _ptr(inter_state_indices), _ptr(o), _stream(stream))
    _raise(st, "gdr_decode_paged")
    return o


# ---------------------------------------------------------------------------
def _gating(q, v, a, b, A_log, dt_bias, eps: float, qk_l2norm: bool, allow_neg_eigval: bool) -> Gating:
    T, HV = q.shape[0], v.shape[1] if v is not None else a.shape[1]
    _check(a, "a", (T, HV), q.dtype)
    _check(b, "b", (T, HV), q.dtype)
    _check(A_log, "A_log", (HV,), torch.float32)
    _check(dt_bias, "dt_bias", (HV,), torch.float32)
    return Gating(a.data_ptr(), b.data_ptr(), A_log.data_ptr(), dt_bias.data_ptr(), float(eps),
                  1 if qk_l2norm else 0, 1 if allow_neg_eigval else 0)


def gdr_gating_prepass(q, k, a, b, A_log, dt_bias, l2norm_eps: float = 1e-6, qk_l2norm: bool = True,
                       allow_neg_eigval: bool = False, q_out=None, k_out=None, g_out=None, beta_out=None,
                       stream=None):
    """Gating front as one pass.  q, k [T, HK, K] raw; a, b [T, HV] (q's dtype); A_log, dt_bias
    [HV] fp32.  Returns (q_out, k_out, g [T, HV] fp32, beta [T, HV]); q_out/k_out may be q/k
    (in place) and are None when qk_l2norm is False."""
    if q.dim() != 3 or a.dim() != 2:
        raise ValueError("q, k are [T, HK, K]; a, b are [T, HV]")
    T, HK, K = q.shape
    HV = a.shape[1]
    _check(q, "q")
    _check(k, "k", (T, HK, K), q.dtype)
    gt = _gating(q, None, a, b, A_log, dt_bias, l2norm_eps, qk_l2norm, allow_neg_eigval)
    if qk_l2norm:
        q_out = torch.empty_like(q) if q_out is None else q_out
        k_out = torch.empty_like(k) if k_out is None else k_out
        _check(q_out, "q_out", (T, HK, K), q.dtype)
        _check(k_out, "k_out", (T, HK, K), q.dtype)
    else:
        q_out = k_out = None
    g_out = torch.empty((T, HV), dtype=torch.float32, device=q.device) if g_out is None else g_out
    beta_out = torch.empty((T, HV), dtype=q.dtype, device=q.device) if beta_out is None else beta_out
    _check(g_out, "g_out", (T, HV), torch.float32)
    _check(beta_out, "beta_out", (T, HV), q.dtype)
    # gdr_problem: V is not read by this pass; K is given as the value width to pass validation
    p = Problem(T, 1, HK, HV, K, K, 1.0, GDR_GATE_SCALAR, _dtype_code(q.dtype))
    st = lib().gdr_gating_prepass(ctypes.byref(p), _ptr(q), _ptr(k), ctypes.byref(gt), _ptr(q_out), _ptr(k_out),
                                  _ptr(g_out), _ptr(beta_out), _stream(stream))
    _raise(st, "gdr_gating_prepass")
    return q_out, k_out, g_out, beta_out


def gdr_decode_paged_gated(q, k, v, a, b, A_log, dt_bias, pool, state_indices, cu_seqlens=None,
                           max_q_len: int = 1, commit: bool = True, inter_states=None, inter_state_indices=None,
                           scale=None, l2norm_eps: float = 1e-6, qk_l2norm: bool = True,
                           allow_neg_eigval: bool = False, o=None, stream=None):
    """gdr_decode_paged with the gating front in the token loop: q, k raw; a, b [T, HV] (q's
    dtype); A_log, dt_bias [HV] fp32.  Returns o."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k are [T, HK, K] and v is [T, HV, V]")
    T, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    _check(q, "q")
    _check(k, "k", (T, HK, K), q.dtype)
    _check(v, "v", (T, HV, V), q.dtype)
    gt = _gating(q, v, a, b, A_log, dt_bias, l2norm_eps, qk_l2norm, allow_neg_eigval)
    _check(state_indices, "state_indices", dtype=torch.int32)
    N = state_indices.shape[0]
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)
    if pool.dim() != 4:
        raise ValueError("pool is [num_slots, HV, V, K]")
    _check(pool, "pool", (pool.shape[0], HV, V, K))
    pool_dt = _dtype_code(pool.dtype)
    ncs = steps = 0
    inter_dt = GDR_F32
    if inter_states is not None:
        if inter_states.dim() != 5:
            raise ValueError("inter_states is [num_cache_slots, cache_steps, HV, V, K]")
        ncs, steps = inter_states.shape[0], inter_states.shape[1]
        _check(inter_states, "inter_states", (ncs, steps, HV, V, K))
        inter_dt = _dtype_code(inter_states.dtype)
        _check(inter_state_indices, "inter_state_indices", (N,), torch.int32)
    if o is None:
        o = torch.empty((T, HV, V), dtype=q.dtype, device=q.device)
    _check(o, "o", (T, HV, V), q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    p = Problem(T, N, HK, HV, K, V, float(scale), GDR_GATE_SCALAR, _dtype_code(q.dtype))
    st = lib().gdr_decode_paged_gated(ctypes.byref(p), int(max_q_len), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(gt),
                                      _ptr(cu_seqlens), _ptr(pool), pool_dt, pool.shape[0], _ptr(state_indices),
                                      1 if commit else 0, _ptr(inter_states), inter_dt, ncs, steps,
                                      _ptr(inter_state_indices), _ptr(o), _stream(stream))
    _raise(st, "gdr_decode_paged_gated")
    return o


def gdr_kda_decode_fused(q, k, v, conv_weight, conv_state, gate_in, gate_weight, A_log, dt_bias, b, pool,
                         state_indices, cu_seqlens=None, max_q_len: int = 1, commit: bool = True, scale=None,
                         conv_bias=None, l2norm_eps: float = 1e-6, norm_weight=None, norm_gate=None,
                         norm_eps: float = 1e-6, o=None, stream=None):
    """Fused KDA decode front (raw q, k, v [T, H, K|V]; conv_weight [C, W]; conv_state
    [slots, C, W-1]; gate_in [T, R]; gate_weight [H*K, R]; A_log [H]; dt_bias [H*K]; b [T, H];
    optional norm_weight [V] with norm_gate [T, H, V]).  Returns o."""
    T, H, K = q.shape
    V = v.shape[2]
    _check(q, "q", (T, H, K))
    _check(k, "k", (T, H, K), q.dtype)
    _check(v, "v", (T, H, V), q.dtype)
    C, W = conv_weight.shape
    assert C == 2 * H * K + H * V, "conv_weight rows: q | k | v channels"
    _check(conv_weight, "conv_weight", (C, W), q.dtype)
    _check(conv_bias, "conv_bias", (C,), q.dtype, optional=True)
    _check(conv_state, "conv_state", (pool.shape[0], C, W - 1), q.dtype, optional=(W == 1))
    R = gate_in.shape[1]
    _check(gate_in, "gate_in", (T, R), q.dtype)
    _check(gate_weight, "gate_weight", (H * K, R), q.dtype)
    _check(A_log, "A_log", (H,), torch.float32)
    _check(dt_bias, "dt_bias", (H * K,), torch.float32)
    _check(b, "b", (T, H), q.dtype)
    _check(norm_weight, "norm_weight", (V,), q.dtype, optional=True)
    _check(norm_gate, "norm_gate", (T, H, V), q.dtype, optional=True)
    N = int(state_indices.shape[0])
    _check(state_indices, "state_indices", (N,), torch.int32)
    _check(pool, "pool", (pool.shape[0], H, V, K))
    if o is None:
        o = torch.empty((T, H, V), dtype=q.dtype, device=q.device)
    _check(o, "o", (T, H, V), q.dtype)
    p = Problem(T, N, H, H, K, V, float(1.0 / math.sqrt(K) if scale is None else scale), GDR_GATE_PER_K,
                _dtype_code(q.dtype))
    f = KdaFront(W, _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), _ptr(gate_in), _ptr(gate_weight), R,
                 _ptr(A_log), _ptr(dt_bias), _ptr(b), float(l2norm_eps), _ptr(norm_weight), _ptr(norm_gate),
                 float(norm_eps))
    st = lib().gdr_kda_decode_fused(ctypes.byref(p), int(max_q_len), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(f),
                                    _ptr(cu_seqlens), _ptr(pool), _dtype_code(pool.dtype), int(pool.shape[0]),
                                    _ptr(state_indices), int(bool(commit)), _ptr(o), _stream(stream))
    _raise(st, "gdr_kda_decode_fused")
    return o
