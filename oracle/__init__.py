"""fp64 CPU oracle of the gated delta-rule recurrence (ctypes front end).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library never imports it, and it imports nothing from the HIP library.

The arithmetic lives in ``gdn_oracle.c`` (plain C, IEEE double, token by
token).  This module only builds/loads it and marshals numpy float64 arrays.
Every function copies its state argument and returns the updated copy, so
callers' arrays are never modified, unless ``inplace=True`` is passed with a
C-contiguous float64 state (large tests use that to avoid copies).

Functions (each cites the page it follows in ``gdn_oracle.c``):
  gdn_step      one decode step, state [B,Hv,Dv,Dk]     (metaltile gated_delta.rs)
  gdn_prefill   varlen prefill over a pool, per token  (pymllm gdn_chunkwise API)
  comba_step    one Comba step, state [B,H,K,V]         (KBench comba_decode_step)
  gates         g (log-space) and beta from a, b        (regolith gdn.metal header)
  conv_silu     4-tap causal conv + SiLU with a rolling history per pool slot
                                                        (regolith gdn.metal conv block)
  gated_rmsnorm y = o rsqrt(mean(o^2) + eps) gamma sigmoid(z) per (token, head)
                                                        (regolith gdn.metal output block)
  gdn_window    T decode tokens per sequence, committing the state after the
                first k (metaltile mt_gated_delta_chunk; regolith commit rule)
  comba_prefill varlen Comba forward over a pool, per token (KBench
                comba_decode_step: the step run over every token)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile ``gdn_oracle.c`` into ``liboracle.so`` with gcc (IEEE double)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_gdn_step.restype = ctypes.c_int
        lib.oracle_gdn_step.argtypes = [_dp] * 7 + [ctypes.c_int] * 5
        lib.oracle_gdn_prefill.restype = ctypes.c_int
        lib.oracle_gdn_prefill.argtypes = (
            [_dp] * 6 + [ctypes.c_int64, _i64p, _i64p, ctypes.c_int, ctypes.c_int64]
            + [ctypes.c_int] * 4 + [ctypes.c_double, ctypes.c_int, ctypes.c_double, _dp])
        lib.oracle_comba_step.restype = ctypes.c_int
        lib.oracle_comba_step.argtypes = [_dp] * 7 + [ctypes.c_double, _dp] + [ctypes.c_int] * 4
        lib.oracle_gates.restype = None
        lib.oracle_gates.argtypes = [_dp] * 6 + [ctypes.c_int64, ctypes.c_int]
        lib.oracle_conv_silu.restype = ctypes.c_int
        lib.oracle_conv_silu.argtypes = [_dp, _dp, _dp, ctypes.c_int64, _i64p, _i64p, ctypes.c_int,
                                         ctypes.c_int64, ctypes.c_int, _dp]
        lib.oracle_gated_rmsnorm.restype = None
        lib.oracle_gated_rmsnorm.argtypes = [_dp, _dp, _dp, ctypes.c_double, ctypes.c_int64,
                                             ctypes.c_int, ctypes.c_int, _dp]
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _state(state, inplace):
    if inplace:
        if not (isinstance(state, np.ndarray) and state.dtype == np.float64
                and state.flags.c_contiguous and state.flags.writeable):
            raise ValueError("inplace=True needs a writeable C-contiguous float64 state")
        return state
    return _f64(state).copy()


def gdn_step(state, q, k, v, g, beta, inplace=False):
    """One decode step.  state [B,Hv,Dv,Dk], q,k [B,Hk,Dk], v [B,Hv,Dv],
    g (log-space) and beta [B,Hv].  Returns (state_new, y) in float64."""
    lib = _load()
    S = _state(state, inplace)
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, Hv, Dv, Dk = S.shape
    Hk = q.shape[1]
    assert q.shape == (B, Hk, Dk) and k.shape == (B, Hk, Dk)
    assert v.shape == (B, Hv, Dv) and g.shape == (B, Hv) and beta.shape == (B, Hv)
    y = np.zeros((B, Hv, Dv), dtype=np.float64)
    rc = lib.oracle_gdn_step(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(y), B, Hk, Hv, Dk, Dv)
    if rc != 0:
        raise ValueError("oracle_gdn_step: invalid shape")
    return S, y


def gdn_prefill(q, k, v, g, beta, pool, cache_indices, cu_seqlens, scale=None,
                l2norm=True, eps=1e-6):
    """Token-by-token varlen prefill.  q,k [T,Hk,Dk], v [T,Hv,Dv], g/beta [T,Hv],
    pool [P,Hv,Dv,Dk].  Returns (pool_new, y) in float64; scale None -> Dk^-1/2."""
    lib = _load()
    P = _f64(pool).copy()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    ci = np.ascontiguousarray(np.asarray(cache_indices, dtype=np.int64))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    N_s = ci.shape[0]
    assert cu.shape == (N_s + 1,)
    if scale is None:
        scale = Dk ** -0.5
    y = np.zeros((T, Hv, Dv), dtype=np.float64)
    rc = lib.oracle_gdn_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(P), P.shape[0],
        ci.ctypes.data_as(_i64p), cu.ctypes.data_as(_i64p), N_s, T, Hk, Hv, Dk, Dv,
        float(scale), 1 if l2norm else 0, float(eps), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_gdn_prefill: invalid shape or index")
    return P, y


def comba_step(state, q, k, v, p, beta, g, scale=None, inplace=False):
    """One Comba step.  state [B,H,K,V]; q,k,p [B,H,K]; v [B,H,V]; beta,g [B,H].
    Returns (state_new, o) in float64; scale None -> K^-1/2."""
    lib = _load()
    S = _state(state, inplace)
    q, k, v, p, beta, g = map(_f64, (q, k, v, p, beta, g))
    B, H, K, V = S.shape
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((B, H, V), dtype=np.float64)
    rc = lib.oracle_comba_step(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(p), _ptr(beta),
                               _ptr(g), float(scale), _ptr(o), B, H, K, V)
    if rc != 0:
        raise ValueError("oracle_comba_step: invalid shape")
    return S, o


def gates(a, b, A_log, dt_bias):
    """g = -exp(A_log) softplus(a + dt_bias) (log-space) and beta = sigmoid(b);
    a, b [T,Hv], A_log and dt_bias [Hv].  Returns (g, beta) in float64."""
    lib = _load()
    a, b, A_log, dt_bias = map(_f64, (a, b, A_log, dt_bias))
    T, Hv = a.shape
    g = np.zeros((T, Hv), dtype=np.float64)
    beta = np.zeros((T, Hv), dtype=np.float64)
    lib.oracle_gates(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(g), _ptr(beta), T, Hv)
    return g, beta


def conv_silu(x, W, hist, cache_indices, cu_seqlens):
    """4-tap causal conv + SiLU per channel with a rolling history.  x [T,C],
    W [C,4] (tap 3 = current token), hist [P,C,3] (oldest first).  Returns
    (out [T,C], hist_new) in float64; hist is not modified."""
    lib = _load()
    x, W = _f64(x), _f64(W)
    H = _f64(hist).copy()
    ci = np.ascontiguousarray(np.asarray(cache_indices, dtype=np.int64))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    T, C = x.shape
    assert W.shape == (C, 4) and H.shape[1:] == (C, 3) and cu.shape == (ci.shape[0] + 1,)
    out = np.zeros((T, C), dtype=np.float64)
    rc = lib.oracle_conv_silu(_ptr(x), _ptr(W), _ptr(H), H.shape[0], ci.ctypes.data_as(_i64p),
                              cu.ctypes.data_as(_i64p), ci.shape[0], T, C, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_conv_silu: invalid shape or index")
    return out, H


def gated_rmsnorm(o, z, gamma, eps=1e-6):
    """y = o rsqrt(mean_j(o^2) + eps) gamma[j] sigmoid(z) over the last axis
    of o, z [T,Hv,Dv]; gamma [Dv].  Returns y in float64."""
    lib = _load()
    o, z, gamma = _f64(o), _f64(z), _f64(gamma)
    T, Hv, Dv = o.shape
    assert z.shape == o.shape and gamma.shape == (Dv,)
    y = np.zeros_like(o)
    lib.oracle_gated_rmsnorm(_ptr(o), _ptr(z), _ptr(gamma), float(eps), T, Hv, Dv, _ptr(y))
    return y


def gdn_window(state, q, k, v, g, beta, commit=None):
    """A decode window of T tokens per sequence: the pinned single step
    (``gdn_step``) applied token by token.  q, k [B,T,Hk,Dk]; v [B,T,Hv,Dv];
    g, beta [B,T,Hv].  Returns (state after the first ``commit`` tokens,
    y [B,T,Hv,Dv]); commit None means all T, 0 returns the state unchanged
    (a verify window), in float64."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T = q.shape[1]
    commit = T if commit is None else int(commit)
    if not 0 <= commit <= T:
        raise ValueError("commit must be in [0, T]")
    S = _f64(state).copy()
    kept = S.copy()
    ys = []
    for t in range(T):
        S, y = gdn_step(S, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t])
        ys.append(y)
        if t + 1 == commit:
            kept = S.copy()
    return kept, np.stack(ys, axis=1)


def comba_prefill(q, k, v, p, beta, g, pool, cache_indices, cu_seqlens, scale=None):
    """Varlen Comba forward over a state pool: the pinned single step
    (``comba_step``) applied token by token to each sequence's slot, as the
    KBench spec describes the forward task (the step run once per token).
    q, k, p [T,H,K]; v [T,H,V]; beta, g [T,H]; pool [P,H,K,V].  Sequence s
    owns tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 and slot cache_indices[s].
    Returns (pool_new, o [T,H,V]) in float64; scale None -> K^-1/2."""
    q, k, v, p, beta, g = map(_f64, (q, k, v, p, beta, g))
    P = _f64(pool).copy()
    ci = np.asarray(cache_indices, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, K = q.shape
    V = v.shape[2]
    if P.ndim != 4 or P.shape[1:] != (H, K, V) or cu.shape != (ci.shape[0] + 1,):
        raise ValueError("comba_prefill: inconsistent shapes")
    if (cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0) or np.any(ci < 0)
            or np.any(ci >= P.shape[0]) or len(set(ci.tolist())) != ci.shape[0]):
        raise ValueError("comba_prefill: invalid cu_seqlens or cache_indices")
    o = np.zeros((T, H, V), dtype=np.float64)
    for s in range(ci.shape[0]):
        S = P[ci[s]][None].copy()
        for t in range(int(cu[s]), int(cu[s + 1])):
            S, ot = comba_step(S, q[t][None], k[t][None], v[t][None], p[t][None], beta[t][None],
                               g[t][None], scale=scale, inplace=True)
            o[t] = ot[0]
        P[ci[s]] = S[0]
    return P, o
