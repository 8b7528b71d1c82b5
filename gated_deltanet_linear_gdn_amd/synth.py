"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the recurrence: it only draws random
tensors with the distributions of the workloads and rounds them to bf16.
Every array it returns is float32 (bf16-representable where the activation
dtype is bf16), int64 for indices; callers move them to the device or hand
them, converted exactly to float64, to the CPU oracle.

Distributions (KBench `comba_decode_step` spec, make_inputs; pymllm
`gdn_chunkwise` parameters for prefill):
  q, v ~ N(0,1); k (and Comba's p) = N(0,1) rows scaled to unit L2 norm;
  beta = sigmoid(U(0,1)); log-gate g = logsigmoid(N(0,1)) / 4 (fp32);
  prefill: q, k, v, a, b ~ N(0,1); A_log ~ U(0, 2.7); dt_bias ~ N(0, 0.5^2).
The generator is numpy PCG64 (``np.random.default_rng(seed)``); each helper
draws its tensors in the order they are listed in its docstring.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = (bits.astype(np.uint32) << 16).view(np.float32)
    return out.reshape(x.shape)


def _unit_rows(z: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(z.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (z / np.maximum(n, 1e-12)).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _logsigmoid(x):
    x = x.astype(np.float64)
    return (np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def _act(x, act: str):
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if act == "bf16" else x


def decode_token(rng, B, Hk, Hv, Dk, Dv, act="bf16"):
    """One decode token: q [B,Hk,Dk], k [B,Hk,Dk] (unit rows), v [B,Hv,Dv],
    beta [B,Hv] (activation dtype), g [B,Hv] (fp32 log-gate)."""
    q = _act(rng.standard_normal((B, Hk, Dk), dtype=np.float32), act)
    k = _act(_unit_rows(rng.standard_normal((B, Hk, Dk), dtype=np.float32)), act)
    v = _act(rng.standard_normal((B, Hv, Dv), dtype=np.float32), act)
    beta = _act(_sigmoid(rng.random((B, Hv), dtype=np.float32)), act)
    g = (_logsigmoid(rng.standard_normal((B, Hv), dtype=np.float32)) / 4.0).astype(np.float32)
    return dict(q=q, k=k, v=v, beta=beta, g=g)


def comba_token(rng, B, H, K, V, act="bf16"):
    """One Comba token: q, k (unit), v, p (unit), beta, g, drawn in the order of
    the KBench generator."""
    q = _act(rng.standard_normal((B, H, K), dtype=np.float32), act)
    k = _act(_unit_rows(rng.standard_normal((B, H, K), dtype=np.float32)), act)
    v = _act(rng.standard_normal((B, H, V), dtype=np.float32), act)
    p = _act(_unit_rows(rng.standard_normal((B, H, K), dtype=np.float32)), act)
    beta = _act(_sigmoid(rng.random((B, H), dtype=np.float32)), act)
    g = (_logsigmoid(rng.standard_normal((B, H), dtype=np.float32)) / 4.0).astype(np.float32)
    return dict(q=q, k=k, v=v, p=p, beta=beta, g=g)


def seq_lengths(rng, n_seq, lo, hi):
    """Sequence lengths drawn uniformly from [lo, hi] (inclusive)."""
    return rng.integers(lo, hi + 1, size=n_seq).astype(np.int64)


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


def prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size, act="bf16"):
    """Packed prefill batch: q, k [T,Hk,Dk]; v [T,Hv,Dv]; a, b [T,Hv]
    (activation dtype, all N(0,1), q/k NOT normalised); A_log [Hv] ~ U(0,2.7);
    dt_bias [Hv] ~ N(0, 0.5^2) (fp32); cache_indices = first N_s entries of a
    random permutation of the pool; cu_seqlens from the lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    q = _act(rng.standard_normal((T, Hk, Dk), dtype=np.float32), act)
    k = _act(rng.standard_normal((T, Hk, Dk), dtype=np.float32), act)
    v = _act(rng.standard_normal((T, Hv, Dv), dtype=np.float32), act)
    a = _act(rng.standard_normal((T, Hv), dtype=np.float32), act)
    b = _act(rng.standard_normal((T, Hv), dtype=np.float32), act)
    A_log = rng.uniform(0.0, 2.7, size=Hv).astype(np.float32)
    dt_bias = (0.5 * rng.standard_normal(Hv, dtype=np.float32)).astype(np.float32)
    cache_indices = rng.permutation(pool_size)[: lengths.shape[0]].astype(np.int64)
    return dict(q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt_bias,
                cache_indices=cache_indices, cu_seqlens=cu_from_lengths(lengths))


def comba_prefill_inputs(rng, lengths, H, K, V, pool_size, act="bf16"):
    """Packed Comba batch with the Comba token distributions: q [T,H,K];
    k [T,H,K] (unit rows); v [T,H,V]; p [T,H,K] (unit rows); beta [T,H]
    (activation dtype); g [T,H] (fp32); cache_indices = first N_s entries of
    a random permutation of the pool; cu_seqlens from the lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    q = _act(rng.standard_normal((T, H, K), dtype=np.float32), act)
    k = _act(_unit_rows(rng.standard_normal((T, H, K), dtype=np.float32)), act)
    v = _act(rng.standard_normal((T, H, V), dtype=np.float32), act)
    p = _act(_unit_rows(rng.standard_normal((T, H, K), dtype=np.float32)), act)
    beta = _act(_sigmoid(rng.random((T, H), dtype=np.float32)), act)
    g = (_logsigmoid(rng.standard_normal((T, H), dtype=np.float32)) / 4.0).astype(np.float32)
    cache_indices = rng.permutation(pool_size)[: lengths.shape[0]].astype(np.int64)
    return dict(q=q, k=k, v=v, p=p, beta=beta, g=g, cache_indices=cache_indices,
                cu_seqlens=cu_from_lengths(lengths))


def layer_inputs(rng, T, Hk, Hv, Dk, Dv, pool_size, act="bf16"):
    """Inputs of the layer steps around the recurrence: qkv [T, C] with
    C = 2*Hk*Dk + Hv*Dv channels ([q heads | k heads | v heads]) ~ N(0,1);
    conv weights [C, 4] ~ N(0, 0.5^2) (fp32); conv history [pool, C, 3] ~
    N(0,1) (fp32); z [T, Hv, Dv] ~ N(0,1); gamma [Dv] ~ 1 + N(0, 0.1^2)
    (fp32).  No trained weights: only the shapes and scales matter here."""
    C = 2 * Hk * Dk + Hv * Dv
    qkv = _act(rng.standard_normal((T, C), dtype=np.float32), act)
    conv_w = (0.5 * rng.standard_normal((C, 4), dtype=np.float32)).astype(np.float32)
    conv_state = rng.standard_normal((pool_size, C, 3), dtype=np.float32)
    z = _act(rng.standard_normal((T, Hv, Dv), dtype=np.float32), act)
    gamma = (1.0 + 0.1 * rng.standard_normal(Dv, dtype=np.float32)).astype(np.float32)
    return dict(qkv=qkv, conv_w=conv_w, conv_state=conv_state, z=z, gamma=gamma)


def layer_decode_inputs(rng, B, Hk, Hv, Dk, Dv, act="bf16"):
    """One decode token of the layer front for B sequences: qkv [B, C] ~
    N(0,1) (C = 2*Hk*Dk + Hv*Dv raw channels, before the conv); conv weights
    [C, 4] ~ N(0, 0.5^2) and conv history [B, C, 3] ~ N(0,1) (fp32); raw
    gates a, b [B, Hv] ~ N(0,1) (activation dtype); A_log [Hv] ~ U(0, 2.7)
    and dt_bias [Hv] ~ N(0, 0.5^2) (fp32): the layer recipe above with the
    prefill's gate recipe."""
    C = 2 * Hk * Dk + Hv * Dv
    qkv = _act(rng.standard_normal((B, C), dtype=np.float32), act)
    conv_w = (0.5 * rng.standard_normal((C, 4), dtype=np.float32)).astype(np.float32)
    conv_state = rng.standard_normal((B, C, 3), dtype=np.float32)
    a = _act(rng.standard_normal((B, Hv), dtype=np.float32), act)
    b = _act(rng.standard_normal((B, Hv), dtype=np.float32), act)
    A_log = rng.uniform(0.0, 2.7, size=Hv).astype(np.float32)
    dt_bias = (0.5 * rng.standard_normal(Hv, dtype=np.float32)).astype(np.float32)
    return dict(qkv=qkv, conv_w=conv_w, conv_state=conv_state, a=a, b=b, A_log=A_log, dt_bias=dt_bias)


# Workload shapes (seed 0 for each).
TINY = dict(B=2, Hk=2, Hv=4, Dk=32, Dv=32, act="f32", prefill_len=16, chunk=8)
DECODE_B64 = dict(B=64, Hk=16, Hv=48, Dk=128, Dv=128, act="bf16")
DECODE_B256 = dict(B=256, Hk=16, Hv=48, Dk=128, Dv=128, act="bf16")
PREFILL_VARLEN = dict(n_seq=8, len_lo=512, len_hi=4096, Hk=16, Hv=48, Dk=128, Dv=128,
                      pool=16, chunk=64, act="bf16")
COMBA_B128 = dict(B=128, H=32, K=128, V=128, act="bf16")
# The Comba decode measure shapes (B, H, K, V) the KBench comba_decode_step
# page lists for its throughput figures (states of 0.47-0.94 GB per copy).
COMBA_MEASURE_SHAPES = ((896, 16, 128, 128), (448, 32, 128, 128), (1792, 8, 128, 128), (1280, 16, 64, 128))
COMBA_PREFILL_VARLEN = dict(n_seq=8, len_lo=512, len_hi=4096, H=32, K=128, V=128, pool=16,
                            chunk=64, act="bf16")
WARMUP_STEPS = 16
