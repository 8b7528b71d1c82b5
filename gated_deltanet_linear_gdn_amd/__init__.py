"""Gated delta-rule (Gated DeltaNet) decode and chunked prefill on MI355X.

Thin Python binding of ``libgdn.so`` (C ABI declared in ``include/gdn.h``).
Each function here has the name of the C entry point it calls and only
marshals arguments: it checks that the torch tensors have the shapes, dtypes,
devices and layouts the C call assumes, allocates outputs that were not
given, and passes raw device pointers plus the current HIP stream.  Every
step of the computation runs in the HIP kernels; there is no fallback.  If
the library has not been built the call raises.

Activation dtype ``act`` follows the tensors: torch.float32 or torch.bfloat16
(q, k, v, p, beta, a, b, y, o all share it).  States are float32, the
log-space gate g is float32.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "GdnError", "library_path", "load_library",
    "gdn_decode_step", "comba_decode_step", "gdn_prefill_gates", "gdn_status_string",
    "gdn_chunk_prefill_workspace", "gdn_chunk_prefill", "gdn_chunk_prefill_raw_workspace", "gdn_chunk_prefill_raw", "gdn_validate_varlen", "GDN_QK_L2NORM", "GDN_KEEP_STATE",
    "gdn_decode_window", "gdn_conv_silu", "gdn_gated_rmsnorm",
    "gdn_chunk_prefill_fixed_workspace", "gdn_chunk_prefill_fixed",
    "comba_chunk_prefill_workspace", "comba_chunk_prefill", "gdn_stream_copy", "gdn_chunk_prefill_noalloc",
    "gdn_conv_decode_step", "gdn_conv_decode_workspace",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn.so")
_lib = None

GDN_F32, GDN_BF16 = 0, 1
_ACT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float


class GdnError(RuntimeError):
    """A libgdn call returned a negative status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {gdn_status_string(status)} ({status})")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgdn.so (once).  torch is imported first so that the library
    binds to the HIP runtime torch already loaded."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m gated_deltanet_linear_gdn_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [_i]
    lib.gdn_decode_step.restype = _i
    lib.gdn_decode_step.argtypes = [_vp] * 8 + [_i] * 6 + [_vp]
    lib.gdn_decode_window.restype = _i
    lib.gdn_decode_window.argtypes = [_vp] * 8 + [_i] * 8 + [_vp]
    lib.comba_decode_step.restype = _i
    lib.comba_decode_step.argtypes = [_vp] * 9 + [_i] * 4 + [_f, _i, _vp]
    lib.gdn_prefill_gates.restype = _i
    lib.gdn_prefill_gates.argtypes = [_vp] * 6 + [_i64, _i, _i, _vp]
    lib.gdn_chunk_prefill_workspace.restype = ctypes.c_size_t
    lib.gdn_chunk_prefill_workspace.argtypes = [_i64, _i, _i, _i, _i, _i, _i, _i]
    lib.gdn_chunk_prefill.restype = _i
    lib.gdn_chunk_prefill.argtypes = ([_vp] * 6 + [_i64, _vp, _vp, _i, _i64] + [_i] * 5
                                      + [_f, ctypes.c_uint, _vp, _i, _vp, ctypes.c_size_t, _vp])
    lib.gdn_chunk_prefill_raw_workspace.restype = ctypes.c_size_t
    lib.gdn_chunk_prefill_raw_workspace.argtypes = [_i64, _i, _i, _i, _i, _i, _i, _i]
    lib.gdn_chunk_prefill_raw.restype = _i
    lib.gdn_chunk_prefill_raw.argtypes = ([_vp] * 8 + [_i64, _vp, _vp, _i, _i64] + [_i] * 5
                                          + [_f, ctypes.c_uint, _vp, _i, _vp, ctypes.c_size_t, _vp])
    lib.gdn_validate_varlen.restype = _i
    lib.gdn_validate_varlen.argtypes = [_vp, _vp, _i, _i64, _i64, _vp]
    lib.gdn_chunk_prefill_gated.restype = _i
    lib.gdn_chunk_prefill_gated.argtypes = ([_vp] * 6 + [_i64, _vp, _vp, _i, _i64] + [_i] * 5
                                            + [_f, ctypes.c_uint, _vp, _vp, _f, _vp, _i, _vp, ctypes.c_size_t, _vp])
    lib.gdn_conv_silu.restype = _i
    lib.gdn_conv_silu.argtypes = [_vp] * 3 + [_i64, _vp, _vp, _i, _i64] + [_i] * 4 + [_vp] * 3 + [_i, _vp]
    lib.gdn_gated_rmsnorm.restype = _i
    lib.gdn_gated_rmsnorm.argtypes = [_vp] * 3 + [_f, _vp, _i64, _i, _i, _i, _vp]
    lib.gdn_chunk_prefill_fixed_workspace.restype = ctypes.c_size_t
    lib.gdn_chunk_prefill_fixed_workspace.argtypes = [_i, _i64, _i, _i, _i, _i, _i, _i]
    lib.gdn_chunk_prefill_fixed.restype = _i
    lib.gdn_chunk_prefill_fixed.argtypes = ([_vp] * 6 + [_i, _i64] + [_i] * 5
                                            + [_f, ctypes.c_uint, _vp, _i, _vp, ctypes.c_size_t, _vp])
    lib.comba_chunk_prefill_workspace.restype = ctypes.c_size_t
    lib.comba_chunk_prefill_workspace.argtypes = [_i64, _i, _i, _i, _i, _i, _i]
    lib.comba_chunk_prefill.restype = _i
    lib.comba_chunk_prefill.argtypes = ([_vp] * 7 + [_i64, _vp, _vp, _i, _i64] + [_i] * 4
                                        + [_f, _vp, _i, _vp, ctypes.c_size_t, _vp])
    lib.gdn_chunk_prefill_noalloc.restype = _i
    lib.gdn_chunk_prefill_noalloc.argtypes = ([_vp] * 6 + [_i64, _vp, _vp, _i, _i64] + [_i] * 5
                                              + [_f, ctypes.c_uint, _vp, _i, _vp])
    lib.gdn_conv_decode_workspace.restype = ctypes.c_size_t
    lib.gdn_conv_decode_workspace.argtypes = [_i] * 5
    lib.gdn_conv_decode_step.restype = _i
    lib.gdn_conv_decode_step.argtypes = [_vp] * 10 + [_i] * 5 + [_f, ctypes.c_uint, _i, _vp, ctypes.c_size_t, _vp]
    lib.gdn_stream_copy.restype = _i
    lib.gdn_conv_prefill_workspace.argtypes = [_i64, _i, _i, _i, _i, _i, _i]
    lib.gdn_conv_prefill_workspace.restype = ctypes.c_size_t
    lib.gdn_conv_prefill.argtypes = ([_vp] * 8 + [_i64, _vp, _vp, _i, _i64] + [_i] * 5
                                     + [_f, ctypes.c_uint, _vp, _vp, _f, _vp, _i, _vp, ctypes.c_size_t, _vp])
    lib.gdn_stream_copy.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
    _lib = lib
    return lib


def gdn_status_string(status: int) -> str:
    return load_library().gdn_status_string(int(status)).decode()


# ------------------------------------------------------------------ helpers


def _stream(device) -> ctypes.c_void_p:
    """The current stream of the tensors' device (the library launches on it,
    with that device current: see _call)."""
    return _vp(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return _vp(t.data_ptr())


def _check(name: str, t: torch.Tensor, shape, dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name}: must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _act_of(t: torch.Tensor) -> int:
    if t.dtype not in _ACT:
        raise TypeError(f"activation dtype {t.dtype} is not float32 or bfloat16")
    return _ACT[t.dtype]


def _call(fn: str, device, *args) -> None:
    """Call entry point fn with `device` current (its kernels launch on the
    current HIP device)."""
    with torch.cuda.device(device):
        rc = getattr(load_library(), fn)(*args)
    if rc != 0:
        raise GdnError(fn, rc)


# ------------------------------------------------------------------ entry points


def gdn_decode_step(state_in, state_out, q, k, v, g, beta, y=None):
    """One decode step (see ``gdn_decode_step`` in include/gdn.h).

    state_in [B,Hv,Dv,Dk] f32; state_out same shape or None (allocated; may be
    state_in itself for an in-place step); q,k [B,Hk,Dk]; v [B,Hv,Dv];
    g [B,Hv] f32 (log gate); beta [B,Hv]; y [B,Hv,Dv] or None.
    Returns (state_out, y)."""
    B, Hv, Dv, Dk = state_in.shape
    Hk = q.shape[1]
    dev = state_in.device
    act = q.dtype
    if state_out is None:
        state_out = torch.empty_like(state_in)
    if y is None:
        y = torch.empty((B, Hv, Dv), dtype=act, device=dev)
    _check("state_in", state_in, (B, Hv, Dv, Dk), torch.float32, dev)
    _check("state_out", state_out, (B, Hv, Dv, Dk), torch.float32, dev)
    _check("q", q, (B, Hk, Dk), act, dev)
    _check("k", k, (B, Hk, Dk), act, dev)
    _check("v", v, (B, Hv, Dv), act, dev)
    _check("g", g, (B, Hv), torch.float32, dev)
    _check("beta", beta, (B, Hv), act, dev)
    _check("y", y, (B, Hv, Dv), act, dev)
    _call("gdn_decode_step", dev, _ptr(state_in), _ptr(state_out), _ptr(q), _ptr(k), _ptr(v),
          _ptr(g), _ptr(beta), _ptr(y), B, Hk, Hv, Dk, Dv, _act_of(q), _stream(dev))
    return state_out, y


def gdn_decode_window(state_in, state_out, q, k, v, g, beta, commit=None, y=None):
    """T decode tokens per sequence with the state kept on chip (see
    ``gdn_decode_window`` in include/gdn.h).  q,k [B,T,Hk,Dk]; v [B,T,Hv,Dv];
    g [B,T,Hv] f32; beta [B,T,Hv]; state_in [B,Hv,Dv,Dk] f32.  state_out
    receives the state after the first ``commit`` tokens (None: all T; 0: a
    verify window that writes no state; state_out None allocates one, or
    pass state_in for in place).  Returns (state_out, y [B,T,Hv,Dv])."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev, act = q.device, q.dtype
    commit = T if commit is None else int(commit)
    if state_out is None and commit > 0:
        state_out = torch.empty_like(state_in)
    if y is None:
        y = torch.empty((B, T, Hv, Dv), dtype=act, device=dev)
    _check("state_in", state_in, (B, Hv, Dv, Dk), torch.float32, dev)
    if state_out is not None:
        _check("state_out", state_out, (B, Hv, Dv, Dk), torch.float32, dev)
    _check("q", q, (B, T, Hk, Dk), act, dev)
    _check("k", k, (B, T, Hk, Dk), act, dev)
    _check("v", v, (B, T, Hv, Dv), act, dev)
    _check("g", g, (B, T, Hv), torch.float32, dev)
    _check("beta", beta, (B, T, Hv), act, dev)
    _check("y", y, (B, T, Hv, Dv), act, dev)
    out_ptr = _ptr(state_out) if state_out is not None else ctypes.c_void_p(0)
    _call("gdn_decode_window", dev, _ptr(state_in), out_ptr, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
          _ptr(y), B, T, Hk, Hv, Dk, Dv, commit, _act_of(q), _stream(dev))
    return state_out, y


def comba_decode_step(state, state_new, q, k, v, p, beta, g, o=None, scale=None):
    """One Comba step (see ``comba_decode_step`` in include/gdn.h).

    state [B,H,K,V] f32; state_new same or None (may be ``state``);
    q,k,p [B,H,K]; v [B,H,V]; beta [B,H]; g [B,H] f32; o [B,H,V] or None;
    scale None -> K^-1/2.  Returns (state_new, o)."""
    B, H, K, V = state.shape
    dev = state.device
    act = q.dtype
    if state_new is None:
        state_new = torch.empty_like(state)
    if o is None:
        o = torch.empty((B, H, V), dtype=act, device=dev)
    _check("state", state, (B, H, K, V), torch.float32, dev)
    _check("state_new", state_new, (B, H, K, V), torch.float32, dev)
    for name, t in (("q", q), ("k", k), ("p", p)):
        _check(name, t, (B, H, K), act, dev)
    _check("v", v, (B, H, V), act, dev)
    _check("beta", beta, (B, H), act, dev)
    _check("g", g, (B, H), torch.float32, dev)
    _check("o", o, (B, H, V), act, dev)
    sc = 0.0 if scale is None else float(scale)
    if scale is not None and not sc > 0.0:
        raise ValueError("scale must be positive (None selects K^-1/2)")
    _call("comba_decode_step", dev, _ptr(state), _ptr(state_new), _ptr(q), _ptr(k), _ptr(v), _ptr(p),
          _ptr(beta), _ptr(g), _ptr(o), B, H, K, V, sc, _act_of(q), _stream(dev))
    return state_new, o


def gdn_prefill_gates(a, b, A_log, dt_bias, g=None, beta=None):
    """g = -exp(A_log) softplus(a + dt_bias) (log-space) and beta = sigmoid(b),
    both [T_tot,Hv] f32 (see ``gdn_prefill_gates`` in include/gdn.h)."""
    T, Hv = a.shape
    dev = a.device
    if g is None:
        g = torch.empty((T, Hv), dtype=torch.float32, device=dev)
    if beta is None:
        beta = torch.empty((T, Hv), dtype=torch.float32, device=dev)
    _check("a", a, (T, Hv), a.dtype, dev)
    _check("b", b, (T, Hv), a.dtype, dev)
    _check("A_log", A_log, (Hv,), torch.float32, dev)
    _check("dt_bias", dt_bias, (Hv,), torch.float32, dev)
    _check("g", g, (T, Hv), torch.float32, dev)
    _check("beta", beta, (T, Hv), torch.float32, dev)
    _call("gdn_prefill_gates", dev, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(g), _ptr(beta),
          T, Hv, _act_of(a), _stream(dev))
    return g, beta


GDN_QK_L2NORM = 1
GDN_KEEP_STATE = 2


def gdn_chunk_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk=64, dtype=None) -> int:
    """Bytes of workspace ``gdn_chunk_prefill`` needs for activations of
    ``dtype`` (torch.bfloat16 by default; 0 for invalid sizes)."""
    act = 0 if dtype == torch.float32 else 1
    return int(load_library().gdn_chunk_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk, act))


def gdn_chunk_prefill(q, k, v, g, beta, state_pool, cache_indices, cu_seqlens, chunk=64,
                      scale=None, l2norm=True, y=None, workspace=None, z=None, gamma=None, eps=1e-6,
                      keep_state=False):
    """Varlen chunkwise prefill, ``state_pool`` updated in place (see
    ``gdn_chunk_prefill`` in include/gdn.h).

    q,k [T,Hk,Dk] raw; v [T,Hv,Dv]; g, beta [T,Hv] f32 (log gate, beta);
    state_pool [P,Hv,Dv,Dk] f32; cache_indices [N_s] int64; cu_seqlens
    [N_s+1] int64 (device tensors, contract not checked here: see
    ``gdn_validate_varlen``); y [T,Hv,Dv] or None; workspace: a uint8 device
    tensor of at least ``gdn_chunk_prefill_workspace`` bytes, or None.
    With z [T,Hv,Dv] and gamma [Dv] f32 given, y is the gated RMS norm of the
    output (``gdn_chunk_prefill_gated``).  keep_state: the pool is only read
    (GDN_KEEP_STATE, a verify window).  Returns y."""
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    P = state_pool.shape[0]
    N_s = cache_indices.shape[0]
    dev = q.device
    act = q.dtype
    if y is None:
        y = torch.empty((T, Hv, Dv), dtype=act, device=dev)
    _check("q", q, (T, Hk, Dk), act, dev)
    _check("k", k, (T, Hk, Dk), act, dev)
    _check("v", v, (T, Hv, Dv), act, dev)
    _check("g", g, (T, Hv), torch.float32, dev)
    _check("beta", beta, (T, Hv), torch.float32, dev)
    _check("state_pool", state_pool, (P, Hv, Dv, Dk), torch.float32, dev)
    _check("cache_indices", cache_indices, (N_s,), torch.int64, dev)
    _check("cu_seqlens", cu_seqlens, (N_s + 1,), torch.int64, dev)
    _check("y", y, (T, Hv, Dv), act, dev)
    need = gdn_chunk_prefill_workspace(T, N_s, Hk, Hv, Dk, Dv, chunk, act)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    sc = 0.0 if scale is None else float(scale)
    flags = (GDN_QK_L2NORM if l2norm else 0) | (GDN_KEEP_STATE if keep_state else 0)
    if z is None and gamma is None:
        _call("gdn_chunk_prefill", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), P,
              _ptr(cache_indices), _ptr(cu_seqlens), N_s, T, Hk, Hv, Dk, Dv, int(chunk), sc,
              flags, _ptr(y), _act_of(q), _ptr(workspace), workspace.numel(), _stream(dev))
        return y
    if z is None or gamma is None:
        raise ValueError("the gated output needs both z and gamma")
    _check("z", z, (T, Hv, Dv), act, dev)
    _check("gamma", gamma, (Dv,), torch.float32, dev)
    _call("gdn_chunk_prefill_gated", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), P,
          _ptr(cache_indices), _ptr(cu_seqlens), N_s, T, Hk, Hv, Dk, Dv, int(chunk), sc, flags,
          _ptr(z), _ptr(gamma), float(eps), _ptr(y), _act_of(q), _ptr(workspace), workspace.numel(),
          _stream(dev))
    return y


def gdn_chunk_prefill_raw_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk=64, dtype=None) -> int:
    """Bytes of workspace ``gdn_chunk_prefill_raw`` needs (torch.bfloat16
    activations by default)."""
    act = 0 if dtype == torch.float32 else 1
    return int(load_library().gdn_chunk_prefill_raw_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk, act))


def gdn_chunk_prefill_raw(q, k, v, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens, chunk=64,
                          scale=None, l2norm=True, y=None, workspace=None, keep_state=False):
    """``gdn_prefill_gates`` and ``gdn_chunk_prefill`` in one call from the
    raw gate inputs (see ``gdn_chunk_prefill_raw`` in include/gdn.h): a, b
    [T,Hv] act, A_log, dt_bias [Hv] f32; the rest as ``gdn_chunk_prefill``.
    Returns y."""
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    P = state_pool.shape[0]
    N_s = cache_indices.shape[0]
    dev, act = q.device, q.dtype
    if y is None:
        y = torch.empty((T, Hv, Dv), dtype=act, device=dev)
    _check("q", q, (T, Hk, Dk), act, dev)
    _check("k", k, (T, Hk, Dk), act, dev)
    _check("v", v, (T, Hv, Dv), act, dev)
    _check("a", a, (T, Hv), act, dev)
    _check("b", b, (T, Hv), act, dev)
    _check("A_log", A_log, (Hv,), torch.float32, dev)
    _check("dt_bias", dt_bias, (Hv,), torch.float32, dev)
    _check("state_pool", state_pool, (P, Hv, Dv, Dk), torch.float32, dev)
    _check("cache_indices", cache_indices, (N_s,), torch.int64, dev)
    _check("cu_seqlens", cu_seqlens, (N_s + 1,), torch.int64, dev)
    _check("y", y, (T, Hv, Dv), act, dev)
    need = gdn_chunk_prefill_raw_workspace(T, N_s, Hk, Hv, Dk, Dv, chunk, act)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    sc = 0.0 if scale is None else float(scale)
    flags = (GDN_QK_L2NORM if l2norm else 0) | (GDN_KEEP_STATE if keep_state else 0)
    _call("gdn_chunk_prefill_raw", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
          _ptr(state_pool), P, _ptr(cache_indices), _ptr(cu_seqlens), N_s, T, Hk, Hv, Dk, Dv, int(chunk), sc,
          flags, _ptr(y), _act_of(q), _ptr(workspace), workspace.numel(), _stream(dev))
    return y


def gdn_conv_decode_workspace(B, Hk, Hv, Dk, Dv) -> int:
    """Bytes of workspace ``gdn_conv_decode_step`` needs."""
    return int(load_library().gdn_conv_decode_workspace(B, Hk, Hv, Dk, Dv))


def gdn_conv_decode_step(state_in, state_out, qkv, conv_w, conv_state, a, b, A_log, dt_bias, Hk, y=None,
                         scale=None, l2norm=True, workspace=None):
    """One decode token of the layer front (see ``gdn_conv_decode_step`` in
    include/gdn.h): conv + SiLU of the raw q/k/v channels with the history
    ``conv_state`` updated in place, q/k L2 norm and scale, gates from raw
    a, b, and the decode step.

    state_in [B,Hv,Dv,Dk] f32; state_out same shape, None (allocated) or
    state_in itself; qkv [B, 2*Hk*Dk + Hv*Dv] act; conv_w [C,4] f32;
    conv_state [B,C,3] f32; a, b [B,Hv] act; A_log, dt_bias [Hv] f32;
    y [B,Hv,Dv] or None; workspace: a uint8 device tensor of at least
    ``gdn_conv_decode_workspace`` bytes, or None.  Returns (state_out, y)."""
    B, Hv, Dv, Dk = state_in.shape
    dev, act = qkv.device, qkv.dtype
    C = 2 * Hk * Dk + Hv * Dv
    if state_out is None:
        state_out = torch.empty_like(state_in)
    if y is None:
        y = torch.empty((B, Hv, Dv), dtype=act, device=dev)
    _check("state_in", state_in, (B, Hv, Dv, Dk), torch.float32, dev)
    _check("state_out", state_out, (B, Hv, Dv, Dk), torch.float32, dev)
    _check("qkv", qkv, (B, C), act, dev)
    _check("conv_w", conv_w, (C, 4), torch.float32, dev)
    _check("conv_state", conv_state, (B, C, 3), torch.float32, dev)
    _check("a", a, (B, Hv), act, dev)
    _check("b", b, (B, Hv), act, dev)
    _check("A_log", A_log, (Hv,), torch.float32, dev)
    _check("dt_bias", dt_bias, (Hv,), torch.float32, dev)
    _check("y", y, (B, Hv, Dv), act, dev)
    need = gdn_conv_decode_workspace(B, Hk, Hv, Dk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    sc = 0.0 if scale is None else float(scale)
    flags = GDN_QK_L2NORM if l2norm else 0
    _call("gdn_conv_decode_step", dev, _ptr(state_in), _ptr(state_out), _ptr(qkv), _ptr(conv_w), _ptr(conv_state),
          _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(y), B, Hk, Hv, Dk, Dv, sc, flags, _act_of(qkv),
          _ptr(workspace), workspace.numel(), _stream(dev))
    return state_out, y


def gdn_chunk_prefill_noalloc(q, k, v, g, beta, state_pool, cache_indices, cu_seqlens, y, chunk=64,
                              scale=None, l2norm=True, keep_state=False):
    """``gdn_chunk_prefill`` with the library's static device workspace
    instead of a caller one (see ``gdn_chunk_prefill_noalloc`` in
    include/gdn.h): nothing is allocated, so y must be given.  Same
    arguments otherwise; calls that overlap in time on one GPU race.
    Returns y."""
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    P = state_pool.shape[0]
    N_s = cache_indices.shape[0]
    dev = q.device
    act = q.dtype
    _check("q", q, (T, Hk, Dk), act, dev)
    _check("k", k, (T, Hk, Dk), act, dev)
    _check("v", v, (T, Hv, Dv), act, dev)
    _check("g", g, (T, Hv), torch.float32, dev)
    _check("beta", beta, (T, Hv), torch.float32, dev)
    _check("state_pool", state_pool, (P, Hv, Dv, Dk), torch.float32, dev)
    _check("cache_indices", cache_indices, (N_s,), torch.int64, dev)
    _check("cu_seqlens", cu_seqlens, (N_s + 1,), torch.int64, dev)
    _check("y", y, (T, Hv, Dv), act, dev)
    sc = 0.0 if scale is None else float(scale)
    flags = (GDN_QK_L2NORM if l2norm else 0) | (GDN_KEEP_STATE if keep_state else 0)
    _call("gdn_chunk_prefill_noalloc", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), P,
          _ptr(cache_indices), _ptr(cu_seqlens), N_s, T, Hk, Hv, Dk, Dv, int(chunk), sc, flags, _ptr(y),
          _act_of(q), _stream(dev))
    return y


def gdn_chunk_prefill_fixed_workspace(B, T, Hk, Hv, Dk, Dv, chunk=64, dtype=None) -> int:
    """Bytes of workspace ``gdn_chunk_prefill_fixed`` needs (torch.bfloat16
    activations by default)."""
    act = 0 if dtype == torch.float32 else 1
    return int(load_library().gdn_chunk_prefill_fixed_workspace(B, T, Hk, Hv, Dk, Dv, chunk, act))


def gdn_chunk_prefill_fixed(q, k, v, g, beta, state, chunk=64, scale=None, l2norm=True, y=None,
                            workspace=None, keep_state=False):
    """Chunkwise prefill of a fixed-length batch, ``state`` updated in place
    (see ``gdn_chunk_prefill_fixed`` in include/gdn.h).  q, k [B,T,Hk,Dk];
    v [B,T,Hv,Dv]; g, beta [B,T,Hv] f32; state [B,Hv,Dv,Dk] f32; y [B,T,Hv,Dv]
    or None.  keep_state: ``state`` is only read (GDN_KEEP_STATE; with no
    norm and scale 1 this is a verify window of T tokens).  Returns y."""
    B, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    dev, act = q.device, q.dtype
    if y is None:
        y = torch.empty((B, T, Hv, Dv), dtype=act, device=dev)
    _check("q", q, (B, T, Hk, Dk), act, dev)
    _check("k", k, (B, T, Hk, Dk), act, dev)
    _check("v", v, (B, T, Hv, Dv), act, dev)
    _check("g", g, (B, T, Hv), torch.float32, dev)
    _check("beta", beta, (B, T, Hv), torch.float32, dev)
    _check("state", state, (B, Hv, Dv, Dk), torch.float32, dev)
    _check("y", y, (B, T, Hv, Dv), act, dev)
    need = gdn_chunk_prefill_fixed_workspace(B, T, Hk, Hv, Dk, Dv, chunk, act)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    sc = 0.0 if scale is None else float(scale)
    _call("gdn_chunk_prefill_fixed", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), B, T,
          Hk, Hv, Dk, Dv, int(chunk), sc, (GDN_QK_L2NORM if l2norm else 0) | (GDN_KEEP_STATE if keep_state else 0),
          _ptr(y), _act_of(q),
          _ptr(workspace), workspace.numel(), _stream(dev))
    return y


def comba_chunk_prefill_workspace(T_tot, N_s, H, K, V, chunk=64) -> int:
    """Bytes of workspace ``comba_chunk_prefill`` needs (bf16 activations)."""
    return int(load_library().comba_chunk_prefill_workspace(T_tot, N_s, H, K, V, chunk, 1))


def comba_chunk_prefill(q, k, v, p, beta, g, state_pool, cache_indices, cu_seqlens, chunk=64,
                        scale=None, o=None, workspace=None):
    """Varlen Comba forward, chunkwise, ``state_pool`` updated in place (see
    ``comba_chunk_prefill`` in include/gdn.h).

    q, k, p [T,H,K] bf16; v [T,H,V] bf16; beta [T,H] bf16; g [T,H] f32;
    state_pool [P,H,K,V] f32; cache_indices [N_s], cu_seqlens [N_s+1] int64
    device tensors; o [T,H,V] bf16 or None; workspace a uint8 device tensor of
    at least ``comba_chunk_prefill_workspace`` bytes, or None.  Returns o."""
    T, H, K = q.shape
    V = v.shape[2]
    P = state_pool.shape[0]
    N_s = cache_indices.shape[0]
    dev, act = q.device, q.dtype
    if o is None:
        o = torch.empty((T, H, V), dtype=act, device=dev)
    for name, t, shape in (("q", q, (T, H, K)), ("k", k, (T, H, K)), ("p", p, (T, H, K)),
                           ("v", v, (T, H, V)), ("beta", beta, (T, H)), ("o", o, (T, H, V))):
        _check(name, t, shape, act, dev)
    _check("g", g, (T, H), torch.float32, dev)
    _check("state_pool", state_pool, (P, H, K, V), torch.float32, dev)
    _check("cache_indices", cache_indices, (N_s,), torch.int64, dev)
    _check("cu_seqlens", cu_seqlens, (N_s + 1,), torch.int64, dev)
    need = comba_chunk_prefill_workspace(T, N_s, H, K, V, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    sc = 0.0 if scale is None else float(scale)
    _call("comba_chunk_prefill", dev, _ptr(q), _ptr(k), _ptr(v), _ptr(p), _ptr(beta), _ptr(g), _ptr(state_pool),
          P, _ptr(cache_indices), _ptr(cu_seqlens), N_s, T, H, K, V, int(chunk), sc, _ptr(o),
          _act_of(q), _ptr(workspace), workspace.numel(), _stream(dev))
    return o


def gdn_conv_silu(qkv, conv_w, conv_state, cache_indices, cu_seqlens, Hk, Hv, Dk, Dv,
                  q=None, k=None, v=None):
    """Layer prologue: 4-tap causal conv + SiLU of the q/k/v channels with the
    per-slot history ``conv_state`` [pool, C, 3] f32 updated in place
    (see ``gdn_conv_silu`` in include/gdn.h).  qkv [T_tot, 2*Hk*Dk + Hv*Dv];
    returns (q [T,Hk,Dk], k [T,Hk,Dk], v [T,Hv,Dv]) in qkv's dtype."""
    T, C = qkv.shape
    dev, dt = qkv.device, qkv.dtype
    if C != 2 * Hk * Dk + Hv * Dv:
        raise ValueError(f"qkv has {C} channels, expected 2*Hk*Dk + Hv*Dv = {2 * Hk * Dk + Hv * Dv}")
    N_s = cache_indices.shape[0]
    q = torch.empty((T, Hk, Dk), dtype=dt, device=dev) if q is None else q
    k = torch.empty((T, Hk, Dk), dtype=dt, device=dev) if k is None else k
    v = torch.empty((T, Hv, Dv), dtype=dt, device=dev) if v is None else v
    _check("qkv", qkv, (T, C), dt, dev)
    _check("conv_w", conv_w, (C, 4), torch.float32, dev)
    _check("conv_state", conv_state, (conv_state.shape[0], C, 3), torch.float32, dev)
    _check("cache_indices", cache_indices, (N_s,), torch.int64, dev)
    _check("cu_seqlens", cu_seqlens, (N_s + 1,), torch.int64, dev)
    _check("q", q, (T, Hk, Dk), dt, dev)
    _check("k", k, (T, Hk, Dk), dt, dev)
    _check("v", v, (T, Hv, Dv), dt, dev)
    _call("gdn_conv_silu", dev, _ptr(qkv), _ptr(conv_w), _ptr(conv_state), conv_state.shape[0],
          _ptr(cache_indices), _ptr(cu_seqlens), N_s, T, Hk, Hv, Dk, Dv, _ptr(q), _ptr(k), _ptr(v),
          _act_of(qkv), _stream(dev))
    return q, k, v


def gdn_conv_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk=64) -> int:
    """Bytes of workspace ``gdn_conv_prefill`` needs (bf16 activations)."""
    return int(load_library().gdn_conv_prefill_workspace(T_tot, N_s, Hk, Hv, Dk, Dv, chunk))


def gdn_conv_prefill(qkv, conv_w, conv_state, a, b, A_log, dt_bias, state_pool, cache_indices, cu_seqlens,
                     Hk, Hv, Dk, Dv, chunk=64, scale=None, l2norm=True, keep_state=False, z=None, gamma=None,
                     eps=1e-6, y=None, workspace=None):
    """The layer's prefill from its raw channels in one call (see
    ``gdn_conv_prefill`` in include/gdn.h): conv + SiLU of qkv [T, C] bf16
    with the history ``conv_state`` [pool, C, 3] f32 updated in place, gates
    from a, b [T,Hv] bf16 and A_log, dt_bias [Hv] f32, the chunked
    recurrence on ``state_pool`` [pool, Hv, Dv, Dk] f32, and the gated norm
    when z [T,Hv,Dv] bf16 and gamma [Dv] f32 are given.  Returns y."""
    T, C = qkv.shape
    dev, act = qkv.device, qkv.dtype
    if C != 2 * Hk * Dk + Hv * Dv:
        raise ValueError(f"qkv has {C} channels, expected 2*Hk*Dk + Hv*Dv = {2 * Hk * Dk + Hv * Dv}")
    P = state_pool.shape[0]
    N_s = cache_indices.shape[0]
    if y is None:
        y = torch.empty((T, Hv, Dv), dtype=act, device=dev)
    _check("qkv", qkv, (T, C), act, dev)
    _check("conv_w", conv_w, (C, 4), torch.float32, dev)
    _check("conv_state", conv_state, (P, C, 3), torch.float32, dev)
    _check("a", a, (T, Hv), act, dev)
    _check("b", b, (T, Hv), act, dev)
    _check("A_log", A_log, (Hv,), torch.float32, dev)
    _check("dt_bias", dt_bias, (Hv,), torch.float32, dev)
    _check("state_pool", state_pool, (P, Hv, Dv, Dk), torch.float32, dev)
    _check("cache_indices", cache_indices, (N_s,), torch.int64, dev)
    _check("cu_seqlens", cu_seqlens, (N_s + 1,), torch.int64, dev)
    _check("y", y, (T, Hv, Dv), act, dev)
    if (z is None) != (gamma is None):
        raise ValueError("z and gamma go together")
    if z is not None:
        _check("z", z, (T, Hv, Dv), act, dev)
        _check("gamma", gamma, (Dv,), torch.float32, dev)
    need = gdn_conv_prefill_workspace(T, N_s, Hk, Hv, Dk, Dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the same device")
    sc = 0.0 if scale is None else float(scale)
    flags = (GDN_QK_L2NORM if l2norm else 0) | (GDN_KEEP_STATE if keep_state else 0)
    zp = None if z is None else _ptr(z)
    gp = None if gamma is None else _ptr(gamma)
    _call("gdn_conv_prefill", dev, _ptr(qkv), _ptr(conv_w), _ptr(conv_state), _ptr(a), _ptr(b), _ptr(A_log),
          _ptr(dt_bias), _ptr(state_pool), P, _ptr(cache_indices), _ptr(cu_seqlens), N_s, T, Hk, Hv, Dk, Dv,
          int(chunk), sc, flags, zp, gp, float(eps), _ptr(y), _act_of(qkv), _ptr(workspace), workspace.numel(),
          _stream(dev))
    return y


def gdn_gated_rmsnorm(o, z, gamma, eps=1e-6, y=None):
    """Layer epilogue: y = o rsqrt(mean(o^2) + eps) gamma sigmoid(z) per
    (token, value head); o, z [T,Hv,Dv], gamma [Dv] f32; y may be o."""
    T, Hv, Dv = o.shape
    dev, dt = o.device, o.dtype
    y = torch.empty_like(o) if y is None else y
    _check("o", o, (T, Hv, Dv), dt, dev)
    _check("z", z, (T, Hv, Dv), dt, dev)
    _check("gamma", gamma, (Dv,), torch.float32, dev)
    _check("y", y, (T, Hv, Dv), dt, dev)
    _call("gdn_gated_rmsnorm", dev, _ptr(o), _ptr(z), _ptr(gamma), float(eps), _ptr(y), T, Hv, Dv,
          _act_of(o), _stream(dev))
    return y


def gdn_validate_varlen(cu_seqlens, cache_indices, T_tot, pool_size) -> int:
    """Check the prefill contract of device ``cu_seqlens``/``cache_indices``
    (synchronises the current stream).  Returns 0 or a negative status."""
    N_s = cache_indices.shape[0]
    dev = cu_seqlens.device
    with torch.cuda.device(dev):
        return int(load_library().gdn_validate_varlen(_ptr(cu_seqlens), _ptr(cache_indices), N_s,
                                                      int(T_tot), int(pool_size), _stream(dev)))


def gdn_stream_copy(src, dst):
    """Measurement helper: copy the bytes of ``src`` into ``dst`` (same
    shape and dtype, contiguous, on one device) with the library's stream
    copy kernel.  Returns dst."""
    _check("dst", dst, tuple(src.shape), src.dtype, src.device)
    if not src.is_contiguous():
        raise ValueError("src: must be contiguous")
    dev = src.device
    _call("gdn_stream_copy", dev, _ptr(src), _ptr(dst), src.numel() * src.element_size(), _stream(dev))
    return dst
