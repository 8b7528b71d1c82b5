"""C-ABI checks that need no GPU: the library loads, exports every function
include/gdn.h declares, and rejects invalid arguments with the documented
status before any HIP call (so nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WORKSPACE, LAUNCH, DEVICE, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    from gated_deltanet_linear_gdn_amd import load_library
    return load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdn_decode_step", "comba_decode_step", "gdn_prefill_gates", "gdn_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    from gated_deltanet_linear_gdn_amd import gdn_status_string
    for code in (OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, WORKSPACE, LAUNCH, DEVICE, ALIAS):
        assert gdn_status_string(code).startswith("GDN_")
    assert gdn_status_string(-1000) == "GDN_ERR_UNKNOWN"


# Fake device addresses: never dereferenced because every call below fails a
# host-side check first.
A = 0x100000
BIG = 1 << 40


def _p(x):
    return ctypes.c_void_p(x)


def decode(lib, state_in=A, state_out=A + BIG, q=A + 2 * BIG, k=A + 3 * BIG, v=A + 4 * BIG,
           g=A + 5 * BIG, beta=A + 6 * BIG, y=A + 7 * BIG, B=2, Hk=2, Hv=4, Dk=128, Dv=128, act=1):
    return lib.gdn_decode_step(_p(state_in), _p(state_out), _p(q), _p(k), _p(v), _p(g), _p(beta),
                               _p(y), B, Hk, Hv, Dk, Dv, act, None)


def test_decode_validation(lib):
    assert decode(lib, B=-1) == SHAPE
    assert decode(lib, Hk=3, Hv=4) == SHAPE
    assert decode(lib, Hk=0) == SHAPE
    assert decode(lib, act=7) == DTYPE
    assert decode(lib, Dk=80) == UNSUP                  # head sizes: multiples of 32 up to 256
    assert decode(lib, Dk=288) == UNSUP
    assert decode(lib, Dv=48) == UNSUP
    assert decode(lib, Dv=288) == UNSUP
    assert decode(lib, q=0) == NULL
    assert decode(lib, state_out=0) == NULL
    assert decode(lib, state_in=A + 4) == ALIGN
    assert decode(lib, k=A + 3 * BIG + 8) == ALIGN
    # partial overlap of the two states, and y inside the state
    assert decode(lib, state_out=A + 4096) == ALIAS
    assert decode(lib, y=A + 64) == ALIAS
    # an input under an output: y over v, q inside the new state
    assert decode(lib, y=A + 4 * BIG + 32) == ALIAS
    assert decode(lib, q=A + BIG + 1024) == ALIAS
    # B == 0 is a no-op that touches nothing, even with null pointers
    assert decode(lib, B=0, q=0, k=0) == OK


def comba(lib, state=A, state_new=A + BIG, q=A + 2 * BIG, k=A + 3 * BIG, v=A + 4 * BIG,
          p=A + 5 * BIG, beta=A + 6 * BIG, g=A + 7 * BIG, o=A + 8 * BIG, B=2, H=2, K=128, V=128,
          scale=0.0, act=1):
    return lib.comba_decode_step(_p(state), _p(state_new), _p(q), _p(k), _p(v), _p(p), _p(beta),
                                 _p(g), _p(o), B, H, K, V, ctypes.c_float(scale), act, None)


def test_comba_validation(lib):
    assert comba(lib, B=-1) == SHAPE
    assert comba(lib, K=0) == SHAPE
    assert comba(lib, act=2) == DTYPE
    assert comba(lib, K=80) == UNSUP
    assert comba(lib, K=256, V=256) == UNSUP            # at most 32 rows of state per thread
    assert comba(lib, K=160, V=160) == UNSUP
    assert comba(lib, p=0) == NULL
    assert comba(lib, o=A + 8 * BIG + 2) == ALIGN
    assert comba(lib, state_new=A + 16) == ALIAS
    assert comba(lib, o=A + 5 * BIG) == ALIAS                     # o over p
    assert comba(lib, H=0, q=0) == OK


def test_gates_validation(lib):
    f = lib.gdn_prefill_gates
    args = [_p(A), _p(A + BIG), _p(A + 2 * BIG), _p(A + 3 * BIG), _p(A + 4 * BIG), _p(A + 5 * BIG)]
    assert f(*args, ctypes.c_int64(-1), 4, 1, None) == SHAPE
    assert f(*args, ctypes.c_int64(8), 0, 1, None) == SHAPE
    assert f(*args, ctypes.c_int64(8), 4, 5, None) == DTYPE
    bad = list(args)
    bad[0] = _p(0)
    assert f(*bad, ctypes.c_int64(8), 4, 1, None) == NULL
    alias = list(args)
    alias[5] = _p(A + 4 * BIG + 4)
    assert f(*alias, ctypes.c_int64(8), 4, 1, None) == ALIAS
    assert f(*bad, ctypes.c_int64(0), 4, 1, None) == OK


def prefill(lib, q=A, k=A + BIG, v=A + 2 * BIG, g=A + 3 * BIG, beta=A + 4 * BIG, pool=A + 5 * BIG,
            P=4, ci=A + 6 * BIG, cu=A + 7 * BIG, N_s=2, T=100, Hk=2, Hv=4, Dk=128, Dv=128, chunk=64,
            flags=1, y=A + 8 * BIG, act=1, ws=A + 9 * BIG, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.gdn_chunk_prefill_workspace(T, N_s, Hk, Hv, Dk, Dv, chunk, act if act in (0, 1) else 1)
    return lib.gdn_chunk_prefill(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(pool), P, _p(ci), _p(cu),
                                 N_s, T, Hk, Hv, Dk, Dv, chunk, ctypes.c_float(0.0), flags, _p(y), act,
                                 _p(ws), ws_bytes, None)


def prefill_raw(lib, q=A, k=A + BIG, v=A + 2 * BIG, a=A + 3 * BIG, b=A + 4 * BIG, A_log=A + 10 * BIG,
                dt_bias=A + 11 * BIG, pool=A + 5 * BIG, P=4, ci=A + 6 * BIG, cu=A + 7 * BIG, N_s=2, T=100, Hk=2,
                Hv=4, Dk=128, Dv=128, chunk=64, flags=1, y=A + 8 * BIG, act=1, ws=A + 9 * BIG, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.gdn_chunk_prefill_raw_workspace(T, N_s, Hk, Hv, Dk, Dv, chunk, act if act in (0, 1) else 1)
    return lib.gdn_chunk_prefill_raw(_p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log), _p(dt_bias), _p(pool), P,
                                     _p(ci), _p(cu), N_s, T, Hk, Hv, Dk, Dv, chunk, ctypes.c_float(0.0), flags,
                                     _p(y), act, _p(ws), ws_bytes, None)


def test_prefill_raw_validation(lib):
    f = lib.gdn_chunk_prefill_raw_workspace
    base = lib.gdn_chunk_prefill_workspace
    assert f(100, 2, 2, 4, 128, 128, 64, 1) == base(100, 2, 2, 4, 128, 128, 64, 1)   # bf16: gates in the WY pass
    assert f(100, 2, 2, 4, 128, 128, 64, 0) >= base(100, 2, 2, 4, 128, 128, 64, 0) + 100 * 4 * 8  # fp32: g, beta
    assert f(100, 2, 2, 4, 128, 128, 48, 0) == 0
    for act in (0, 1):
        assert prefill_raw(lib, act=act, a=0) == NULL
        assert prefill_raw(lib, act=act, dt_bias=0) == NULL
        assert prefill_raw(lib, act=act, a=A + 8 * BIG + 64) == ALIAS      # a over y
        assert prefill_raw(lib, act=act, b=A + 9 * BIG) == ALIAS           # b over the workspace
        assert prefill_raw(lib, act=act, flags=4) == UNSUP
        assert prefill_raw(lib, act=act, ws_bytes=1024) == WORKSPACE
        assert prefill_raw(lib, act=act, N_s=0, q=0, a=0) == OK            # nothing to do
    assert prefill_raw(lib, act=9) == DTYPE


def test_prefill_workspace_size(lib):
    f = lib.gdn_chunk_prefill_workspace
    for act in (0, 1):
        assert f(100, 2, 2, 4, 128, 128, 64, act) > 0
        assert f(100, 2, 2, 4, 128, 128, 48, act) == 0          # unsupported chunk
        assert f(-1, 2, 2, 4, 128, 128, 64, act) == 0
        # grows with tokens, sequences and heads
        assert f(1000, 2, 2, 4, 128, 128, 64, act) > f(100, 2, 2, 4, 128, 128, 64, act)
        assert f(100, 20, 2, 4, 128, 128, 64, act) > f(100, 2, 2, 4, 128, 128, 64, act)
        assert f(100, 2, 2, 8, 128, 128, 64, act) > f(100, 2, 2, 4, 128, 128, 64, act)
    assert f(100, 2, 2, 4, 128, 128, 64, 7) == 0                 # unknown dtype
    # bf16 builds T and P on chip: no per-chunk matrices in the workspace
    assert f(1000, 2, 2, 4, 128, 128, 64, 1) < f(1000, 2, 2, 4, 128, 128, 64, 0)
    # Dk > 128 runs 32-token chunks whatever chunk asks for
    assert f(1000, 2, 2, 4, 256, 128, 64, 1) == f(1000, 2, 2, 4, 128, 128, 32, 1)
    assert f(1000, 2, 2, 4, 160, 128, 64, 1) == f(1000, 2, 2, 4, 128, 128, 32, 1)
    assert f(1000, 2, 2, 4, 96, 128, 64, 1) == f(1000, 2, 2, 4, 128, 128, 64, 1)
    assert f(1000, 2, 2, 4, 256, 128, 16, 1) == f(1000, 2, 2, 4, 128, 128, 16, 1)


def test_prefill_validation(lib):
    assert prefill(lib, N_s=-1) == SHAPE
    assert prefill(lib, Hk=3) == SHAPE
    assert prefill(lib, act=9) == DTYPE
    assert prefill(lib, Dk=512) == UNSUP
    assert prefill(lib, Dk=256, act=0) == UNSUP            # Dk > 128 with bf16 activations only
    assert prefill(lib, Dk=160, act=0) == UNSUP
    assert prefill(lib, Dk=80) == UNSUP                    # a multiple of 32 up to 256
    assert prefill(lib, Dv=40) == UNSUP
    assert prefill(lib, chunk=128) == UNSUP
    assert prefill(lib, flags=4) == UNSUP                 # no such flag
    assert prefill(lib, flags=3, ws=0) == NULL            # GDN_QK_L2NORM | GDN_KEEP_STATE pass the flag check
    assert prefill(lib, ws=0) == NULL
    assert prefill(lib, cu=0) == NULL
    assert prefill(lib, q=0) == NULL
    assert prefill(lib, pool=A + 5 * BIG + 8) == ALIGN
    assert prefill(lib, v=A + 2 * BIG + 2) == ALIGN
    assert prefill(lib, Hv=65536, Hk=65536, Dv=256) == UNSUP  # 64 tokens of v span >= 1 GiB
    assert prefill(lib, ws_bytes=1024) == WORKSPACE
    assert prefill(lib, y=A + 5 * BIG + 64) == ALIAS      # y inside the pool
    assert prefill(lib, y=A + 2 * BIG + 64) == ALIAS      # y over v (an input)
    assert prefill(lib, ws=A + 4 * BIG) == ALIAS          # workspace over beta
    assert prefill(lib, q=A + 5 * BIG) == ALIAS           # an input inside the pool
    assert prefill(lib, N_s=0, q=0, cu=0) == OK           # nothing to do


def test_validate_varlen_rejects_before_any_copy(lib):
    f = lib.gdn_validate_varlen
    assert f(_p(A), _p(A + BIG), -1, 10, 4, None) == SHAPE
    assert f(_p(0), _p(A + BIG), 2, 10, 4, None) == NULL
    assert f(_p(A), _p(A + BIG), 0, 0, 4, None) == OK
    assert f(_p(A), _p(A + BIG), 0, 5, 4, None) == SHAPE


def conv(lib, x=A, w=A + BIG, hist=A + 2 * BIG, P=4, ci=A + 3 * BIG, cu=A + 4 * BIG, N_s=2, T=100,
         Hk=2, Hv=4, Dk=128, Dv=128, q=A + 5 * BIG, k=A + 6 * BIG, v=A + 7 * BIG, act=1):
    return lib.gdn_conv_silu(_p(x), _p(w), _p(hist), P, _p(ci), _p(cu), N_s, T, Hk, Hv, Dk, Dv,
                             _p(q), _p(k), _p(v), act, None)


def test_conv_silu_validation(lib):
    # every check returns before any HIP call (fake device addresses)
    assert conv(lib, N_s=-1) == SHAPE
    assert conv(lib, Hk=0) == SHAPE
    assert conv(lib, act=7) == DTYPE
    assert conv(lib, Dk=100) == UNSUP      # channels per head not a multiple of 8
    assert conv(lib, x=0) == NULL
    assert conv(lib, hist=0) == NULL
    assert conv(lib, q=A + 5 * BIG + 2) == ALIGN
    assert conv(lib, k=A + 5 * BIG + 16) == ALIAS   # k overlaps q
    assert conv(lib, v=A + 2) == ALIGN
    assert conv(lib, v=A + 16) == ALIAS             # v overlaps qkv
    assert conv(lib, N_s=0, x=0) == OK              # nothing to do
    assert conv(lib, T=0, x=0) == OK


def norm(lib, o=A, z=A + BIG, gamma=A + 2 * BIG, eps=1e-6, y=A + 3 * BIG, T=10, Hv=4, Dv=128, act=1):
    return lib.gdn_gated_rmsnorm(_p(o), _p(z), _p(gamma), ctypes.c_float(eps), _p(y), T, Hv, Dv, act, None)


def test_gated_rmsnorm_validation(lib):
    assert norm(lib, T=-1) == SHAPE
    assert norm(lib, eps=-1.0) == SHAPE
    assert norm(lib, act=3) == DTYPE
    assert norm(lib, Dv=96) == UNSUP
    assert norm(lib, z=0) == NULL
    assert norm(lib, gamma=A + 2 * BIG + 4) == ALIGN
    assert norm(lib, y=A + BIG + 16) == ALIAS       # y overlaps z
    assert norm(lib, y=A + 16) == ALIAS             # partial overlap with o
    assert norm(lib, T=0, o=0) == OK


def test_gated_prefill_validation(lib):
    def gated(z=A + 10 * BIG, gamma=A + 11 * BIG, eps=1e-6, Dv=128, y=A + 8 * BIG, N_s=2, T=100):
        ws = lib.gdn_chunk_prefill_workspace(T, N_s, 2, 4, 128, Dv, 64, 1)
        return lib.gdn_chunk_prefill_gated(
            _p(A), _p(A + BIG), _p(A + 2 * BIG), _p(A + 3 * BIG), _p(A + 4 * BIG), _p(A + 5 * BIG), 4,
            _p(A + 6 * BIG), _p(A + 7 * BIG), N_s, T, 2, 4, 128, Dv, 64, ctypes.c_float(0.0), 1,
            _p(z), _p(gamma), ctypes.c_float(eps), _p(y), 1, _p(A + 9 * BIG), ws, None)
    assert gated(eps=-1.0) == SHAPE
    assert gated(Dv=96) == UNSUP
    assert gated(z=0) == NULL
    assert gated(gamma=0) == NULL
    assert gated(z=A + 10 * BIG + 8) == ALIGN
    assert gated(z=A + 8 * BIG + 16) == ALIAS        # z overlaps y
    assert gated(z=A + 5 * BIG + 64) == ALIAS        # z overlaps the state pool
    assert gated(N_s=0, z=0) == OK


def test_decode_window_validation(lib):
    def win(sin=A, sout=A + BIG, q=A + 2 * BIG, k=A + 3 * BIG, v=A + 4 * BIG, g=A + 5 * BIG,
            beta=A + 6 * BIG, y=A + 7 * BIG, B=4, T=4, Hk=2, Hv=4, Dk=128, Dv=128, commit=4, act=1):
        return lib.gdn_decode_window(_p(sin), _p(sout), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(y),
                                     B, T, Hk, Hv, Dk, Dv, commit, act, None)
    assert win(T=0) == SHAPE
    assert win(commit=5) == SHAPE
    assert win(commit=-1) == SHAPE
    assert win(T=9, commit=2) == UNSUP
    assert win(act=2) == DTYPE
    assert win(sout=0) == NULL                   # committing needs state_out
    assert win(sout=0, commit=0, B=0) == OK
    assert win(q=A + 2 * BIG + 4) == ALIGN
    assert win(sout=A + 64) == ALIAS             # partial overlap with state_in
    assert win(y=A + 16) == ALIAS
    assert win(y=A + 3 * BIG) == ALIAS           # y over k
    assert win(g=A + BIG + 256) == ALIAS         # g inside the committed state


def test_comba_prefill_validation(lib):
    def cp(q=A, k=A + BIG, v=A + 2 * BIG, p=A + 3 * BIG, beta=A + 4 * BIG, g=A + 5 * BIG,
           pool=A + 6 * BIG, ci=A + 7 * BIG, cu=A + 8 * BIG, o=A + 9 * BIG, ws=A + 10 * BIG,
           N_s=2, T=100, H=4, K=128, V=128, chunk=64, act=1, ws_bytes=None, P=4):
        if ws_bytes is None:
            ws_bytes = lib.comba_chunk_prefill_workspace(T, N_s, H, K, V, chunk, 1)
        return lib.comba_chunk_prefill(_p(q), _p(k), _p(v), _p(p), _p(beta), _p(g), _p(pool), P, _p(ci),
                                       _p(cu), N_s, T, H, K, V, chunk, ctypes.c_float(0.0), _p(o), act,
                                       _p(ws), ws_bytes, None)
    f = lib.comba_chunk_prefill_workspace
    assert f(100, 2, 4, 128, 128, 64, 1) == lib.gdn_chunk_prefill_workspace(100, 2, 4, 4, 128, 128, 64, 1)
    assert f(100, 2, 4, 128, 128, 64, 0) == 0            # bf16 activations only
    assert f(100, 2, 4, 128, 128, 48, 1) == 0
    assert cp(N_s=-1) == SHAPE
    assert cp(H=0) == SHAPE
    assert cp(act=9) == DTYPE
    assert cp(act=0) == UNSUP                             # fp32 activations
    assert cp(K=512) == UNSUP
    assert cp(V=40) == UNSUP
    assert cp(chunk=128) == UNSUP
    assert cp(p=0) == NULL
    assert cp(ws=0) == NULL
    assert cp(p=A + 3 * BIG + 8) == ALIGN
    assert cp(pool=A + 6 * BIG + 4) == ALIGN
    assert cp(ws_bytes=1024) == WORKSPACE
    assert cp(o=A + 6 * BIG + 64) == ALIAS                # o inside the pool
    assert cp(ws=A + 9 * BIG + 64) == ALIAS               # workspace inside o
    assert cp(o=A + 3 * BIG) == ALIAS                     # o over p (an input)
    assert cp(beta=A + 10 * BIG) == ALIAS                 # an input inside the workspace
    assert cp(N_s=0, q=0, p=0) == OK


def test_fixed_prefill_validation(lib):
    f = lib.gdn_chunk_prefill_fixed_workspace
    # the varlen workspace for B sequences of T tokens plus the index arrays
    assert f(4, 100, 2, 4, 128, 128, 64, 1) > lib.gdn_chunk_prefill_workspace(400, 4, 2, 4, 128, 128, 64, 1)
    assert f(4, 100, 2, 4, 128, 128, 48, 1) == 0
    assert f(-1, 100, 2, 4, 128, 128, 64, 1) == 0

    def fx(state=A + 5 * BIG, y=A + 8 * BIG, ws=A + 9 * BIG, B=4, T=100, Hk=2, Hv=4, Dk=128, Dv=128,
           chunk=64, act=1, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = f(B, T, Hk, Hv, Dk, Dv, chunk, 1)
        return lib.gdn_chunk_prefill_fixed(_p(A), _p(A + BIG), _p(A + 2 * BIG), _p(A + 3 * BIG),
                                           _p(A + 4 * BIG), _p(state), B, T, Hk, Hv, Dk, Dv, chunk,
                                           ctypes.c_float(0.0), 1, _p(y), act, _p(ws), ws_bytes, None)
    assert fx(B=-1) == SHAPE
    assert fx(Hk=3) == SHAPE
    assert fx(act=5) == DTYPE
    assert fx(B=0, ws=0) == OK
    assert fx(T=0, ws=0) == OK
    assert fx(ws=0) == NULL
    assert fx(chunk=48, ws_bytes=1 << 30) == UNSUP
    assert fx(Dk=512, ws_bytes=1 << 30) == UNSUP
    assert fx(ws_bytes=1024) == WORKSPACE
    assert fx(ws=A + 9 * BIG + 8) == ALIGN
    main = lib.gdn_chunk_prefill_workspace(400, 4, 2, 4, 128, 128, 64, 1)
    assert fx(ws=A + 5 * BIG - main) == ALIAS        # index arrays at the start of the state
    assert fx(y=A + 5 * BIG + 64) == ALIAS           # y inside the state (varlen check)
    assert fx(ws=A + 4 * BIG - main) == ALIAS        # index arrays over beta


def test_stream_copy_validation(lib):
    cp = lambda src=A, dst=A + BIG, n=4096: lib.gdn_stream_copy(_p(src), _p(dst), n, None)
    assert cp(n=0, src=0, dst=0) == OK          # nothing to copy: no pointer is used
    assert cp(src=0) == NULL
    assert cp(dst=0) == NULL
    assert cp(src=A + 8) == ALIGN
    assert cp(n=4100) == SHAPE
    assert cp(dst=A + 2048) == ALIAS
    assert cp(dst=A + (1 << 44), n=(1 << 31) * 4096) == UNSUP  # more workgroups than one launch holds


def prefill_noalloc(lib, q=A, k=A + BIG, v=A + 2 * BIG, g=A + 3 * BIG, beta=A + 4 * BIG, pool=A + 5 * BIG,
                    P=4, ci=A + 6 * BIG, cu=A + 7 * BIG, N_s=2, T=100, Hk=2, Hv=4, Dk=128, Dv=128, chunk=64,
                    flags=1, y=A + 8 * BIG, act=1):
    return lib.gdn_chunk_prefill_noalloc(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(pool), P, _p(ci), _p(cu),
                                         N_s, T, Hk, Hv, Dk, Dv, chunk, ctypes.c_float(0.0), flags, _p(y), act,
                                         None)


def test_prefill_noalloc_validation(lib):
    """The caller's arguments are checked, and a call whose workspace would
    exceed the library's 128 MiB scratch is refused, before any HIP call."""
    assert prefill_noalloc(lib, N_s=-1) == SHAPE
    assert prefill_noalloc(lib, act=9) == DTYPE
    assert prefill_noalloc(lib, Dk=512) == UNSUP
    assert prefill_noalloc(lib, q=0) == NULL
    assert prefill_noalloc(lib, cu=0) == NULL
    assert prefill_noalloc(lib, pool=A + 5 * BIG + 8) == ALIGN
    assert prefill_noalloc(lib, y=A + 5 * BIG + 64) == ALIAS
    assert prefill_noalloc(lib, N_s=0, q=0, cu=0) == OK
    big = dict(T=20000, N_s=8, Hk=16, Hv=48)
    assert lib.gdn_chunk_prefill_workspace(20000, 8, 16, 48, 128, 128, 64, 1) > 128 << 20
    assert prefill_noalloc(lib, **big) == WORKSPACE
    assert lib.gdn_chunk_prefill_workspace(8000, 8, 16, 48, 128, 128, 64, 1) <= 128 << 20


def conv_decode(lib, s_in=A, s_out=A + BIG, x=A + 2 * BIG, w=A + 3 * BIG, hist=A + 4 * BIG, a=A + 6 * BIG,
                b=A + 7 * BIG, alog=A + 8 * BIG, dtb=A + 9 * BIG, y=A + 10 * BIG, B=2, Hk=2, Hv=4, Dk=128,
                Dv=128, flags=1, act=1, ws=A + 11 * BIG, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.gdn_conv_decode_workspace(B, Hk, Hv, Dk, Dv)
    return lib.gdn_conv_decode_step(_p(s_in), _p(s_out), _p(x), _p(w), _p(hist), _p(a), _p(b), _p(alog),
                                    _p(dtb), _p(y), B, Hk, Hv, Dk, Dv, ctypes.c_float(0.0), flags, act, _p(ws),
                                    ws_bytes, None)


def test_conv_decode_validation(lib):
    assert lib.gdn_conv_decode_workspace(256, 16, 48, 128, 128) == 256 * (2 * 16 * 128 + 48 * 128 + 96) * 4
    assert lib.gdn_conv_decode_workspace(-1, 16, 48, 128, 128) == 0
    assert conv_decode(lib, B=-1) == SHAPE
    assert conv_decode(lib, Hk=3) == SHAPE
    assert conv_decode(lib, act=5) == DTYPE
    assert conv_decode(lib, Dk=80) == UNSUP
    assert conv_decode(lib, Dv=48) == UNSUP
    assert conv_decode(lib, flags=4) == UNSUP
    assert conv_decode(lib, B=0, x=0) == OK               # nothing to do
    assert conv_decode(lib, x=0) == NULL
    assert conv_decode(lib, hist=0) == NULL
    assert conv_decode(lib, ws=0) == NULL
    assert conv_decode(lib, s_in=A + 8) == ALIGN
    assert conv_decode(lib, w=A + 3 * BIG + 4) == ALIGN
    assert conv_decode(lib, hist=A + 4 * BIG + 2) == ALIGN
    assert conv_decode(lib, ws=A + 11 * BIG + 8) == ALIGN
    assert conv_decode(lib, ws_bytes=100) == WORKSPACE
    assert conv_decode(lib, s_out=A + 64) == ALIAS        # partial overlap of the states
    assert conv_decode(lib, y=A + 2 * BIG) == ALIAS       # y over the raw channels
    assert conv_decode(lib, hist=A + BIG + 128) == ALIAS  # history inside the new state
    assert conv_decode(lib, ws=A + 4 * BIG + 64) == ALIAS # workspace over the history


def conv_prefill(lib, x=A, w=A + BIG, hist=A + 2 * BIG, a=A + 3 * BIG, b=A + 4 * BIG, A_log=A + 5 * BIG,
                 dtb=A + 6 * BIG, pool=A + 7 * BIG, P=4, ci=A + 8 * BIG, cu=A + 9 * BIG, N_s=2, T=100, Hk=2,
                 Hv=4, Dk=128, Dv=128, chunk=64, flags=1, z=0, gamma=0, eps=1e-6, y=A + 10 * BIG, act=1,
                 ws=A + 11 * BIG, ws_bytes=1 << 30):
    return lib.gdn_conv_prefill(_p(x), _p(w), _p(hist), _p(a), _p(b), _p(A_log), _p(dtb), _p(pool), P, _p(ci),
                                _p(cu), N_s, T, Hk, Hv, Dk, Dv, chunk, 0.0, flags, _p(z), _p(gamma), eps, _p(y),
                                act, _p(ws), ws_bytes, None)


def test_conv_prefill_validation(lib):
    f = lib.gdn_conv_prefill_workspace
    base = lib.gdn_chunk_prefill_workspace(100, 2, 2, 4, 128, 128, 64, 1)
    # the prefill's workspace, then the convolved q, k, v (bf16), each 256-byte aligned
    assert f(100, 2, 2, 4, 128, 128, 64) == base + 2 * 51200 + 102400 + 256
    assert f(100, 2, 2, 4, 128, 128, 48) == 0
    assert f(-1, 2, 2, 4, 128, 128, 64) == 0
    assert conv_prefill(lib, N_s=-1) == SHAPE
    assert conv_prefill(lib, Hk=3) == SHAPE
    assert conv_prefill(lib, act=7) == DTYPE
    assert conv_prefill(lib, act=0) == UNSUP                     # bf16 activations only
    assert conv_prefill(lib, Dk=80) == UNSUP
    assert conv_prefill(lib, chunk=48) == UNSUP
    assert conv_prefill(lib, flags=4) == UNSUP
    assert conv_prefill(lib, z=A + 12 * BIG, gamma=A + 13 * BIG, Dv=96) == UNSUP   # the norm: Dv a power of two
    assert conv_prefill(lib, z=A + 12 * BIG, gamma=A + 13 * BIG, eps=-1.0) == SHAPE
    assert conv_prefill(lib, N_s=0, x=0, ws=0) == OK             # nothing to do
    assert conv_prefill(lib, x=0) == NULL
    assert conv_prefill(lib, hist=0) == NULL
    assert conv_prefill(lib, a=0) == NULL
    assert conv_prefill(lib, ws=0) == NULL
    assert conv_prefill(lib, z=A + 12 * BIG) == NULL              # z without gamma
    assert conv_prefill(lib, x=A + 8) == ALIGN
    assert conv_prefill(lib, w=A + BIG + 4) == ALIGN
    assert conv_prefill(lib, hist=A + 2 * BIG + 8) == ALIGN
    assert conv_prefill(lib, ws_bytes=base) == WORKSPACE        # no room for the convolved rows
    assert conv_prefill(lib, y=A + 64) == ALIAS                  # y over the raw channels
    assert conv_prefill(lib, hist=A + 7 * BIG + 256) == ALIAS    # history inside the pool
    assert conv_prefill(lib, a=A + 2 * BIG + 64) == ALIAS        # a raw gate under the history
    assert conv_prefill(lib, w=A + 11 * BIG + base + 512) == ALIAS   # weights under the convolved rows
    ws_total = f(100, 2, 2, 4, 128, 128, 64)
    assert conv_prefill(lib, y=A + 11 * BIG + ws_total - 256) == ALIAS  # y over the workspace's last bytes
