"""Seeded synthetic inputs for the gated-delta-rule workloads.

This module only draws random numbers and lays them out; it holds none of the
recurrence's arithmetic.  Both the HIP path and the CPU oracle are fed from the
arrays built here, so they see the same bytes.

Input contract (FlashQLA PR #1 "Fused recurrent GDN decode + SGLang DFlash
verify kernel", verify-kernel commit): q and k arrive l2-normalised per
(token, head); g and beta arrive already activated.  g is the natural-log decay,
finite and <= 0.

Workloads (sizes as named in the problem statement of the build):

* ``tiny``       1 sequence, T=64, 2 heads, K=V=64, fp32 I/O, zero initial state.
* ``decode``     256 sequences, q_len 1, 16 key / 32 value heads, K=V=128, bf16
                 I/O, fp32 paged pool [1024, 32, 128, 128] ~ N(0, 0.1); 26 of the
                 256 state indices are -1 (padding); commit.
* ``verify``     64 sequences of 12 tokens (cu_seqlens = 12*arange(65)), same
                 heads, bf16 pool, bf16 per-token intermediate buffer, no commit.
* ``prefill``    8 ragged sequences summing to 32768 tokens (two of length 64 and
                 65), 32 heads, K=V=128, bf16, fp32 initial state ~ N(0, 0.1).
* ``long_batch`` 4 sequences of 16384 tokens, 16 heads, K=V=128, bf16, fp32 initial state
                 (few long sequences: the segmented route of the chunked forward).
* ``kda``        1 sequence of 65536+37 tokens, 16 heads, per-channel decay gk
                 (50% U[-2,0], 25% exactly 0, 25% exactly -2), beta 25% 0 /
                 25% 1 / 50% sigmoid(N(0,1)), zero initial state.

Every array is numpy; bf16 tensors are carried as ``uint16`` bit patterns
(round-to-nearest-even from fp32).  ``widen`` turns any of them into float64
exactly.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 (exact)."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(x: np.ndarray) -> np.ndarray:
    """Exact widening of an fp32 array or a bf16 bit-pattern array to float64."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def cast_io(x32: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    return f32_to_bf16_bits(x32) if dtype == BF16 else x32


def _l2norm_rows(x: np.ndarray) -> np.ndarray:
    """Normalise the last axis to unit length in fp32 (the upstream input contract)."""
    x = x.astype(np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-6))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


@dataclasses.dataclass
class Problem:
    """One set of inputs plus metadata.  Shapes (packed varlen, contiguous):

    q, k  [T, HK, K]      v  [T, HV, V]      g  [T, HV] (scalar) or [T, HV, K] (per-K)
    beta  [T, HV]         cu_seqlens int32 [N+1]
    initial_state float32 [N, HV, V, K] or None (zeros)
    Paged extras: pool [num_slots, HV, V, K] (pool_dtype), state_indices int32 [N],
    inter_state_indices int32 [N], cache shape (num_cache_slots, cache_steps).
    """
    name: str
    T: int
    N: int
    HK: int
    HV: int
    K: int
    V: int
    io_dtype: str
    per_k_gate: bool
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    initial_state: Optional[np.ndarray] = None
    # paged decode / verify
    pool: Optional[np.ndarray] = None
    pool_dtype: Optional[str] = None
    state_indices: Optional[np.ndarray] = None
    commit: bool = False
    inter_dtype: Optional[str] = None
    inter_state_indices: Optional[np.ndarray] = None
    num_cache_slots: int = 0
    cache_steps: int = 0
    max_q_len: int = 1

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))


def _qkv(rng, T, HK, HV, K, V, io_dtype):
    q = _l2norm_rows(rng.standard_normal((T, HK, K), dtype=np.float32))
    k = _l2norm_rows(rng.standard_normal((T, HK, K), dtype=np.float32))
    v = rng.standard_normal((T, HV, V), dtype=np.float32)
    return cast_io(q, io_dtype), cast_io(k, io_dtype), cast_io(v, io_dtype)


def _beta_sigmoid(rng, T, HV, io_dtype):
    return cast_io(_sigmoid(rng.standard_normal((T, HV), dtype=np.float32)), io_dtype)


def dense_problem(seed: int, lengths, HK: int, HV: int, K: int, V: int, io_dtype: str = BF16,
                  g_range=(-0.1, 0.0), g_endpoints: float = 0.0, per_k_gate: bool = False,
                  beta_mode: str = "sigmoid", with_initial_state: bool = True,
                  state_std: float = 0.1, name: str = "dense") -> Problem:
    """Generic packed-varlen problem used by the dense recurrent and chunked entries.

    g_endpoints = p puts a fraction p of the gates exactly at each end of g_range
    (the adversarial gate-endpoint cases); beta_mode "mixed" draws 25% exact 0,
    25% exact 1 and 50% sigmoid(N(0,1)).
    """
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    T = int(sum(lengths))
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    q, k, v = _qkv(rng, T, HK, HV, K, V, io_dtype)
    gshape = (T, HV, K) if per_k_gate else (T, HV)
    lo, hi = g_range
    g = rng.uniform(lo, hi, size=gshape).astype(np.float32)
    if g_endpoints > 0:
        u = rng.uniform(0.0, 1.0, size=gshape)
        g[u < g_endpoints] = np.float32(hi)
        g[u > 1.0 - g_endpoints] = np.float32(lo)
    if beta_mode == "sigmoid":
        beta = _beta_sigmoid(rng, T, HV, io_dtype)
    elif beta_mode == "mixed":
        b = _sigmoid(rng.standard_normal((T, HV), dtype=np.float32))
        u = rng.uniform(0.0, 1.0, size=(T, HV))
        b[u < 0.25] = 0.0
        b[(u >= 0.25) & (u < 0.5)] = 1.0
        beta = cast_io(b, io_dtype)
    elif beta_mode == "one":
        beta = cast_io(np.ones((T, HV), np.float32), io_dtype)
    elif beta_mode == "zero":
        beta = cast_io(np.zeros((T, HV), np.float32), io_dtype)
    else:
        raise ValueError(beta_mode)
    h0 = None
    if with_initial_state:
        h0 = (rng.standard_normal((N, HV, V, K), dtype=np.float32) * np.float32(state_std)).astype(np.float32)
    return Problem(name=name, T=T, N=N, HK=HK, HV=HV, K=K, V=V, io_dtype=io_dtype,
                   per_k_gate=per_k_gate, scale=1.0 / math.sqrt(K), q=q, k=k, v=v, g=g,
                   beta=beta, cu_seqlens=cu, initial_state=h0)


def ragged_lengths(seed: int, n: int = 8, total: int = 32768, lo: int = 1, hi: int = 8192,
                   fixed=(64, 65)) -> list:
    """Ragged lengths: n draws in U[lo, hi]; two positions overwritten with the fixed
    lengths; the others rescaled so the sum is ``total`` (rounding residual on the
    largest); order shuffled."""
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=n).astype(np.float64)
    free = n - len(fixed)
    rest = x[:free]
    target = total - sum(fixed)
    scaled = np.maximum(1, np.rint(rest * (target / rest.sum()))).astype(np.int64)
    scaled[np.argmax(scaled)] += target - int(scaled.sum())
    out = list(int(s) for s in scaled) + list(fixed)
    perm = rng.permutation(n)
    return [out[i] for i in perm]


def tiny(seed: int = 1) -> Problem:
    """1 sequence, T=64, 2 heads, K=V=64, fp32, g ~ U[-0.05, 0], zero initial state."""
    p = dense_problem(seed, [64], HK=2, HV=2, K=64, V=64, io_dtype=F32, g_range=(-0.05, 0.0),
                      with_initial_state=False, name="tiny")
    return p


def prefill(seed: int = 4, adversarial: bool = False, lengths=None, HV: int = 32, HK: Optional[int] = None) -> Problem:
    """Ragged GDN prefill: 8 sequences, 32768 tokens, 32 heads, K=V=128, bf16."""
    if lengths is None:
        lengths = ragged_lengths(seed)
    HK = HV if HK is None else HK
    if adversarial:
        return dense_problem(seed, lengths, HK=HK, HV=HV, K=128, V=128, io_dtype=BF16,
                             g_range=(-2.0, 0.0), g_endpoints=0.25, name="prefill_adv")
    return dense_problem(seed, lengths, HK=HK, HV=HV, K=128, V=128, io_dtype=BF16,
                         g_range=(-0.1, 0.0), name="prefill")


def long_batch(seed: int = 6, N: int = 4, length: int = 16384, HV: int = 16) -> Problem:
    """A few long GDN sequences with few heads (the case the segmented route exists for): 4 x 16384
    tokens, 16 heads, K=V=128, bf16, g ~ U[-0.1, 0], fp32 initial state."""
    return dense_problem(seed, [length] * N, HK=HV, HV=HV, K=128, V=128, io_dtype=BF16,
                         g_range=(-0.1, 0.0), name="long_batch")


def kda(seed: int = 5, T: int = 65536 + 37, HV: int = 16) -> Problem:
    """KDA per-channel decay stress: one long sequence, per-K log-decay, mixed beta."""
    return dense_problem(seed, [T], HK=HV, HV=HV, K=128, V=128, io_dtype=BF16,
                         g_range=(-2.0, 0.0), g_endpoints=0.25, per_k_gate=True,
                         beta_mode="mixed", with_initial_state=False, name="kda")


def kda_overflow_case(seed: int = 105, T: int = 200, HV: int = 2) -> Problem:
    """All gk = -2 and beta = 1: a 64-token chunk reaches a log-decay prefix of -128,
    which a factor exp(-prefix) cannot represent in fp32 (cuLA PR #113 review)."""
    p = dense_problem(seed, [T], HK=HV, HV=HV, K=128, V=128, io_dtype=BF16, per_k_gate=True,
                      beta_mode="one", with_initial_state=False, name="kda_overflow")
    p.g[...] = np.float32(-2.0)
    return p


def paged_problem(seed: int, B: int, q_len: int, HK: int, HV: int, K: int, V: int,
                  num_slots: int, pool_dtype: str, io_dtype: str = BF16, pad_count: int = 0,
                  commit: bool = True, inter_dtype: Optional[str] = None,
                  g_range=(-1.0, 0.0), ragged: bool = False, per_k_gate: bool = False,
                  state_std: float = 0.1, name: str = "paged", cache_steps: Optional[int] = None,
                  with_cu_seqlens: Optional[bool] = None) -> Problem:
    """Paged decode / verify problem.  ``ragged`` draws per-sequence q_len in 1..q_len."""
    rng = np.random.default_rng(seed)
    if ragged:
        lengths = rng.integers(1, q_len + 1, size=B)
    else:
        lengths = np.full(B, q_len, dtype=np.int64)
    T = int(lengths.sum())
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    q, k, v = _qkv(rng, T, HK, HV, K, V, io_dtype)
    gshape = (T, HV, K) if per_k_gate else (T, HV)
    g = rng.uniform(g_range[0], g_range[1], size=gshape).astype(np.float32)
    beta = _beta_sigmoid(rng, T, HV, io_dtype)
    pool32 = rng.standard_normal((num_slots, HV, V, K), dtype=np.float32)
    pool32 *= np.float32(state_std)
    pool = cast_io(pool32, pool_dtype)
    del pool32
    idx = rng.choice(num_slots, size=B, replace=False).astype(np.int32)
    if pad_count:
        pads = rng.choice(B, size=pad_count, replace=False)
        idx[pads] = -1
    p = Problem(name=name, T=T, N=B, HK=HK, HV=HV, K=K, V=V, io_dtype=io_dtype,
                per_k_gate=per_k_gate, scale=1.0 / math.sqrt(K), q=q, k=k, v=v, g=g, beta=beta,
                cu_seqlens=cu, pool=pool, pool_dtype=pool_dtype, state_indices=idx, commit=commit,
                max_q_len=int(lengths.max()) if B else 1)
    if with_cu_seqlens is None:
        with_cu_seqlens = not (q_len == 1 and not ragged)
    p._use_cu = with_cu_seqlens  # type: ignore[attr-defined]
    if inter_dtype is not None:
        p.inter_dtype = inter_dtype
        p.cache_steps = cache_steps if cache_steps is not None else q_len
        p.num_cache_slots = B + 1
        p.inter_state_indices = np.arange(B, dtype=np.int32)
    return p


def decode(seed: int = 2, B: int = 256, num_slots: int = 1024) -> Problem:
    """q_len 1 decode: fp32 pool, 10% (rounded) of the state indices are -1, commit."""
    return paged_problem(seed, B=B, q_len=1, HK=16, HV=32, K=128, V=128, num_slots=num_slots,
                         pool_dtype=F32, pad_count=int(round(0.1 * B)), commit=True, name="decode")


def verify(seed: int = 3, B: int = 64, num_slots: int = 1024, pad: bool = False) -> Problem:
    """Speculative verify: 12 tokens per sequence, bf16 pool, bf16 per-token states, no commit."""
    return paged_problem(seed, B=B, q_len=12, HK=16, HV=32, K=128, V=128, num_slots=num_slots,
                         pool_dtype=BF16, pad_count=int(round(0.1 * B)) if pad else 0, commit=False,
                         inter_dtype=BF16, cache_steps=12, name="verify")


@dataclasses.dataclass
class RawGating:
    """Raw inputs of the gating front (for the gated entry points), drawn only:

    q, k     [T, HK, K] io dtype, NOT normalised (N(0,1) rows times a per-row length
             in U[0.25, 4], so the normalisation changes them)
    a, b     [T, HV] io dtype: the decay and beta inputs before softplus / sigmoid
    A_log    [HV] fp32 (log of U[1, 16]);  dt_bias [HV] fp32 (U[-7, -2])
    eps      added to the sum of squares under the square root of the normalisation
    allow_neg_eigval  beta doubled
    A fraction ``over_threshold`` of the a values is set to 25 so a + dt_bias exceeds the
    softplus threshold 20 and the pass-through branch is exercised.
    """
    q: np.ndarray
    k: np.ndarray
    a: np.ndarray
    b: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    eps: float
    qk_l2norm: bool
    allow_neg_eigval: bool


def raw_gating(seed: int, T: int, HK: int, HV: int, K: int, io_dtype: str = BF16,
               allow_neg_eigval: bool = False, qk_l2norm: bool = True, eps: float = 1e-6,
               over_threshold: float = 0.02) -> RawGating:
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, HK, K), dtype=np.float32) * rng.uniform(0.25, 4.0, (T, HK, 1)).astype(np.float32)
    k = rng.standard_normal((T, HK, K), dtype=np.float32) * rng.uniform(0.25, 4.0, (T, HK, 1)).astype(np.float32)
    a = rng.standard_normal((T, HV), dtype=np.float32)
    if over_threshold > 0:
        a[rng.uniform(0.0, 1.0, (T, HV)) < over_threshold] = np.float32(25.0)
    b = (rng.standard_normal((T, HV), dtype=np.float32) * np.float32(1.5)).astype(np.float32)
    A_log = np.log(rng.uniform(1.0, 16.0, HV)).astype(np.float32)
    dt_bias = rng.uniform(-7.0, -2.0, HV).astype(np.float32)
    return RawGating(q=cast_io(q, io_dtype), k=cast_io(k, io_dtype), a=cast_io(a, io_dtype),
                     b=cast_io(b, io_dtype), A_log=A_log, dt_bias=dt_bias, eps=float(eps),
                     qk_l2norm=bool(qk_l2norm), allow_neg_eigval=bool(allow_neg_eigval))


@dataclasses.dataclass
class KdaFrontProblem:
    """Inputs of the fused KDA decode front (raw projections, convolution, gate, paged state):

    q, k [T, H, K], v [T, H, V] io dtype (raw, before the convolution); conv_weight [C, W],
    conv_bias [C] or None, conv_state [slots, C, W-1] io dtype with C = 2HK + HV (q | k | v);
    gate_in [T, R], gate_weight [H*K, R] io dtype; A_log [H], dt_bias [H*K] fp32; b [T, H];
    norm_weight [V] and norm_gate [T, H, V] io dtype (or None: no epilogue); pool
    [slots, H, V, K] (pool_dtype); state_indices int32 [N] with -1 for padded sequences."""
    T: int
    N: int
    H: int
    K: int
    V: int
    R: int
    W: int
    io_dtype: str
    pool_dtype: str
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    conv_weight: np.ndarray
    conv_bias: Optional[np.ndarray]
    conv_state: np.ndarray
    gate_in: np.ndarray
    gate_weight: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    b: np.ndarray
    norm_weight: Optional[np.ndarray]
    norm_gate: Optional[np.ndarray]
    pool: np.ndarray
    state_indices: np.ndarray
    cu_seqlens: np.ndarray
    max_q_len: int
    l2_eps: float = 1e-6
    norm_eps: float = 1e-6


def kda_front_problem(seed: int, B: int, q_len: int, H: int, K: int = 128, V: int = 128, R: int = 128,
                      W: int = 4, num_slots: Optional[int] = None, io_dtype: str = BF16, pool_dtype: str = F32,
                      pad_count: int = 0, ragged: bool = False, with_bias: bool = True,
                      with_epilogue: bool = True) -> KdaFrontProblem:
    """Seeded draws: raw q, k, v ~ N(0, 1); taps ~ N(0, 0.5^2), bias ~ N(0, 0.1^2); windows ~ N(0, 1);
    gate input ~ N(0, 1) and projection ~ N(0, 1/R) (unit-variance projections); A_log = ln U[1, 16];
    dt_bias ~ U[-5, -1]; b ~ N(0, 1.5^2); norm weight ~ U[0.5, 1.5], norm gate ~ N(0, 1); state pool
    ~ N(0, 0.1^2); distinct slots, pad_count of them -1."""
    rng = np.random.default_rng(seed)
    num_slots = num_slots if num_slots is not None else max(2 * B, 4)
    lengths = rng.integers(1, q_len + 1, size=B) if ragged else np.full(B, q_len, dtype=np.int64)
    T = int(lengths.sum())
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    C = 2 * H * K + H * V
    f = lambda *shape: rng.standard_normal(shape, dtype=np.float32)
    q = cast_io(f(T, H, K), io_dtype)
    k = cast_io(f(T, H, K), io_dtype)
    v = cast_io(f(T, H, V), io_dtype)
    conv_weight = cast_io(f(C, W) * np.float32(0.5), io_dtype)
    conv_bias = cast_io(f(C) * np.float32(0.1), io_dtype) if with_bias else None
    conv_state = cast_io(f(num_slots, C, W - 1), io_dtype)
    gate_in = cast_io(f(T, R), io_dtype)
    gate_weight = cast_io(f(H * K, R) * np.float32(1.0 / math.sqrt(R)), io_dtype)
    A_log = np.log(rng.uniform(1.0, 16.0, H)).astype(np.float32)
    dt_bias = rng.uniform(-5.0, -1.0, H * K).astype(np.float32)
    b = cast_io(f(T, H) * np.float32(1.5), io_dtype)
    norm_weight = cast_io(rng.uniform(0.5, 1.5, V).astype(np.float32), io_dtype) if with_epilogue else None
    norm_gate = cast_io(f(T, H, V), io_dtype) if with_epilogue else None
    pool = cast_io(f(num_slots, H, V, K) * np.float32(0.1), pool_dtype)
    idx = rng.choice(num_slots, size=B, replace=False).astype(np.int32)
    if pad_count:
        idx[rng.choice(B, size=pad_count, replace=False)] = -1
    return KdaFrontProblem(T=T, N=B, H=H, K=K, V=V, R=R, W=W, io_dtype=io_dtype, pool_dtype=pool_dtype,
                           scale=1.0 / math.sqrt(K), q=q, k=k, v=v, conv_weight=conv_weight, conv_bias=conv_bias,
                           conv_state=conv_state, gate_in=gate_in, gate_weight=gate_weight, A_log=A_log,
                           dt_bias=dt_bias, b=b, norm_weight=norm_weight, norm_gate=norm_gate, pool=pool,
                           state_indices=idx, cu_seqlens=cu, max_q_len=int(lengths.max()) if B else 1)
