"""GPU parity of gdn_decode_step against the fp64 oracle (through the C ABI).

Tolerances: state max relative error <= 1e-5; y <= 1e-5 when fp32, and when
bf16 element by element (tests.helpers.check_bf16_out: relative Frobenius
<= 2e-2, max |error| <= 1e-2 of the largest value, per row <= 2e-2; y is
rounded to bf16 once, ~2e-3 at most).
"""
import numpy as np
import pytest
import torch

import oracle
import gated_deltanet_linear_gdn_amd as gdn
from gated_deltanet_linear_gdn_amd import synth
from tests.helpers import check_bf16_out, maxrel, relF, to_dev, to_np, oracle_decode_batched

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _dev_token(tok, act):
    d = DT[act]
    return dict(q=to_dev(tok["q"], d, DEV), k=to_dev(tok["k"], d, DEV), v=to_dev(tok["v"], d, DEV),
                beta=to_dev(tok["beta"], d, DEV), g=to_dev(tok["g"], torch.float32, DEV))


def _step(S_dev, t, out=None):
    return gdn.gdn_decode_step(S_dev, out, t["q"], t["k"], t["v"], t["g"], t["beta"])


def _check_y(y_gpu, y_ref, act):
    if act == "f32":
        assert maxrel(y_gpu, y_ref) <= 1e-5
    else:
        check_bf16_out(y_gpu, y_ref, "y")


def test_tiny_fp32_from_zero_then_steps():
    """Tiny fp32 workload: B=2, Hk=2, Hv=4, Dk=Dv=32, zero state, then 4 more steps."""
    c = synth.TINY
    rng = np.random.default_rng(0)
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    S_ref = np.zeros((B, Hv, Dv, Dk))
    S_dev = torch.zeros((B, Hv, Dv, Dk), dtype=torch.float32, device=DEV)
    for step in range(5):
        tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv, act="f32")
        S_dev, y = _step(S_dev, _dev_token(tok, "f32"))
        S_ref, y_ref = oracle.gdn_step(S_ref, tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"])
        assert maxrel(to_np(S_dev), S_ref) <= 1e-5, step
        assert maxrel(to_np(y), y_ref) <= 1e-5, step


SHAPES = [
    # B, Hk, Hv, Dk, Dv
    (3, 1, 3, 32, 32),
    (2, 2, 6, 64, 96),
    (3, 2, 4, 128, 128),
    (1, 1, 2, 128, 160),   # Dv not a multiple of the rows a workgroup covers
    (2, 3, 3, 256, 64),
    (1, 1, 1, 256, 256),
    (5, 4, 8, 128, 32),
    (2, 1, 48, 32, 32),    # 48 value heads read one key head
    (1, 6, 48, 64, 64),    # groups of 8
    # head sizes that are multiples of 32 but not powers of two (lanes past
    # the row's columns idle)
    (2, 2, 4, 96, 64),
    (2, 1, 2, 160, 96),
    (1, 2, 4, 192, 128),
    (2, 1, 3, 224, 160),
]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("B,Hk,Hv,Dk,Dv", SHAPES)
def test_parity_shapes(B, Hk, Hv, Dk, Dv, act):
    rng = np.random.default_rng(B * 1000 + Dk + Dv)
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv, act=act)
    S_dev, y = _step(to_dev(S0, torch.float32, DEV), _dev_token(tok, act))
    S_ref, y_ref = oracle.gdn_step(S0, tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"])
    assert maxrel(to_np(S_dev), S_ref) <= 1e-5
    _check_y(to_np(y), y_ref, act)


def test_in_place_equals_out_of_place_and_is_deterministic():
    rng = np.random.default_rng(11)
    B, Hk, Hv, Dk, Dv = 4, 2, 8, 128, 128
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    t = _dev_token(synth.decode_token(rng, B, Hk, Hv, Dk, Dv), "bf16")
    S_a, y_a = _step(to_dev(S0, torch.float32, DEV), t)
    S_b, y_b = _step(to_dev(S0, torch.float32, DEV), t)
    S_c = to_dev(S0, torch.float32, DEV)
    S_c2, y_c = _step(S_c, t, out=S_c)
    assert S_c2.data_ptr() == S_c.data_ptr()
    assert torch.equal(S_a, S_b) and torch.equal(y_a, y_b)
    assert torch.equal(S_a, S_c) and torch.equal(y_a, y_c)


def test_head_sharing_matches_expanded_keys_bitwise():
    """Contiguous key-head sharing: repeating q/k to Hv heads gives identical bits."""
    rng = np.random.default_rng(12)
    B, Hk, Hv, Dk, Dv = 2, 2, 6, 128, 64
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv)
    t = _dev_token(tok, "bf16")
    S1, y1 = _step(to_dev(S0, torch.float32, DEV), t)
    t2 = dict(t)
    t2["q"] = t["q"].repeat_interleave(Hv // Hk, dim=1).contiguous()
    t2["k"] = t["k"].repeat_interleave(Hv // Hk, dim=1).contiguous()
    S2, y2 = _step(to_dev(S0, torch.float32, DEV), t2)
    assert torch.equal(S1, S2) and torch.equal(y1, y2)


def test_beta_zero_is_pure_decay_on_gpu():
    rng = np.random.default_rng(13)
    B, Hk, Hv, Dk, Dv = 2, 1, 2, 128, 128
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv, act="f32")
    tok["beta"] = np.zeros_like(tok["beta"])
    S_dev, _ = _step(to_dev(S0, torch.float32, DEV), _dev_token(tok, "f32"))
    ref = np.exp(tok["g"].astype(np.float64))[:, :, None, None] * S0
    assert maxrel(to_np(S_dev), ref) <= 1e-6


def _warm_state(rng, B, Hk, Hv, Dk, Dv, steps=synth.WARMUP_STEPS):
    """State after `steps` oracle decode steps from zero (bf16 activations),
    handed over as float32."""
    S = np.zeros((B, Hv, Dv, Dk))
    for _ in range(steps):
        S, _ = oracle_decode_batched(S, synth.decode_token(rng, B, Hk, Hv, Dk, Dv))
    return S.astype(np.float32)


def test_decode_batch_b64_full_tensor():
    """Qwen-style decode batch: B=64, Hk=16, Hv=48, Dk=Dv=128, warmed 16 steps;
    three GPU steps checked on the full state and output."""
    c = synth.DECODE_B64
    rng = np.random.default_rng(0)
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    S = _warm_state(rng, B, Hk, Hv, Dk, Dv)
    S_dev = to_dev(S, torch.float32, DEV)
    S_ref = S.astype(np.float64)
    for _ in range(3):
        tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv)
        S_dev, y = _step(S_dev, _dev_token(tok, "bf16"))
        S_ref, y_ref = oracle_decode_batched(S_ref, tok)
        assert maxrel(to_np(S_dev), S_ref) <= 1e-5
        _check_y(to_np(y), y_ref, "bf16")


def test_decode_batch_b256():
    """Large decode batch B=256 (0.8 GB state) in the benchmark's launch
    configuration (functional ping-pong).  Step 1 is checked on the whole
    state and output; the oracle then follows 8 sampled sequences through
    3 more steps.  The warmed state is 16 oracle-warmed sequences tiled over
    the batch."""
    c = synth.DECODE_B256
    rng = np.random.default_rng(0)
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    W = _warm_state(rng, 16, Hk, Hv, Dk, Dv)
    S = np.tile(W, (B // 16, 1, 1, 1))
    bufs = [to_dev(S, torch.float32, DEV), torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=DEV)]
    sample = np.array([0, 1, 37, 100, 128, 201, 254, 255])
    S_full = S.astype(np.float64)
    del S
    for step in range(4):
        tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv)
        t = _dev_token(tok, "bf16")
        _, y = gdn.gdn_decode_step(bufs[step % 2], bufs[(step + 1) % 2], t["q"], t["k"], t["v"],
                                   t["g"], t["beta"])
        if step == 0:
            S_full, y_ref = oracle_decode_batched(S_full, tok)
            assert maxrel(to_np(bufs[1]), S_full) <= 1e-5
            _check_y(to_np(y), y_ref, "bf16")
            S_ref = S_full[sample].copy()
            del S_full
            continue
        sub = {n: a[sample] for n, a in tok.items()}
        S_ref, y_ref = oracle_decode_batched(S_ref, sub)
        got = bufs[(step + 1) % 2][torch.from_numpy(sample).to(DEV)]
        assert maxrel(to_np(got), S_ref) <= 1e-5, step
        _check_y(to_np(y)[sample], y_ref, "bf16")


def test_decode_batch_b256_sampled_through_1000_steps():
    """The benchmark's launch configuration for its 1,000 timed steps: B=256,
    16 token sets used cyclically, functional ping-pong.  The oracle follows
    8 sampled sequences (384 (b, hv) slices) through every step; their state
    and y are checked every 250 steps, so error that builds up over the run
    would show."""
    c = synth.DECODE_B256
    rng = np.random.default_rng(7)
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    W = _warm_state(rng, 16, Hk, Hv, Dk, Dv)
    S = np.tile(W, (B // 16, 1, 1, 1))
    sample = np.array([0, 5, 64, 100, 129, 190, 222, 255])
    S_ref = S[sample].astype(np.float64)
    bufs = [to_dev(S, torch.float32, DEV), torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=DEV)]
    del S
    toks = [synth.decode_token(rng, B, Hk, Hv, Dk, Dv) for _ in range(16)]
    dtoks = [_dev_token(t, "bf16") for t in toks]
    subs = [{n: a[sample] for n, a in t.items()} for t in toks]
    y = torch.empty((B, Hv, Dv), dtype=torch.bfloat16, device=DEV)
    idx = torch.from_numpy(sample).to(DEV)
    for step in range(1000):
        t = dtoks[step % 16]
        gdn.gdn_decode_step(bufs[step % 2], bufs[(step + 1) % 2], t["q"], t["k"], t["v"], t["g"], t["beta"], y)
        S_ref, y_ref = oracle_decode_batched(S_ref, subs[step % 16])
        if (step + 1) % 250 == 0:
            torch.cuda.synchronize()
            print(f"b256 long run: step {step + 1}", flush=True)
            assert maxrel(to_np(bufs[(step + 1) % 2][idx]), S_ref) <= 1e-5, step
            _check_y(to_np(y)[sample], y_ref, "bf16")


def test_batch_beyond_one_launch_grid():
    """65,538 sequences: more than one launch's grid holds (65,535 sequences),
    so the batch runs in two slices.  The oracle follows the sequences on both
    sides of the seam and at the ends, for one step and for a 2-token window."""
    rng = np.random.default_rng(41)
    B, Hk, Hv, Dk, Dv = 65538, 1, 2, 32, 32
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk), dtype=np.float32)).astype(np.float32)
    tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv)
    sample = np.array([0, 1, 30000, 65533, 65534, 65535, 65536, 65537])
    S_dev, y = _step(to_dev(S0, torch.float32, DEV), _dev_token(tok, "bf16"))
    S_ref, y_ref = oracle_decode_batched(S0[sample].astype(np.float64), {n: a[sample] for n, a in tok.items()})
    idx = torch.from_numpy(sample).to(DEV)
    assert maxrel(to_np(S_dev[idx]), S_ref) <= 1e-5
    _check_y(to_np(y)[sample], y_ref, "bf16")
    del S_dev, y
    w = _window_tokens(rng, B, 2, Hk, Hv, Dk, Dv, "bf16")
    dw = {n: to_dev(x, torch.float32 if n == "g" else torch.bfloat16, DEV) for n, x in w.items()}
    s_io = to_dev(S0, torch.float32, DEV)
    _, yw = gdn.gdn_decode_window(s_io, s_io, dw["q"], dw["k"], dw["v"], dw["g"], dw["beta"])
    torch.cuda.synchronize()
    Sw, yw_ref = oracle.gdn_window(S0[sample], *(w[n][sample] for n in ("q", "k", "v", "g", "beta")))
    assert maxrel(to_np(s_io[idx]), Sw) <= 1e-5
    check_bf16_out(to_np(yw)[sample], yw_ref, "window y")


# ------------------------------------------------------------ decode windows

WINDOW_CASES = [
    # B, T, Hk, Hv, Dk, Dv, commit, act
    (3, 1, 1, 3, 32, 32, 1, "f32"),
    (2, 3, 2, 6, 64, 96, 2, "bf16"),
    (3, 4, 2, 4, 128, 128, 4, "bf16"),
    (2, 4, 2, 4, 128, 128, 0, "bf16"),       # verify: no state write
    (1, 8, 1, 2, 128, 160, 5, "f32"),        # Dv not a multiple of a workgroup's rows
    (2, 8, 1, 1, 256, 64, 8, "bf16"),
    (2, 3, 1, 2, 96, 64, 2, "bf16"),
    (1, 4, 1, 2, 224, 96, 4, "f32"),
]


def _window_tokens(rng, B, T, Hk, Hv, Dk, Dv, act):
    toks = [synth.decode_token(rng, B, Hk, Hv, Dk, Dv, act=act) for _ in range(T)]
    return {n: np.stack([t[n] for t in toks], axis=1) for n in toks[0]}


@pytest.mark.parametrize("B,T,Hk,Hv,Dk,Dv,commit,act", WINDOW_CASES)
def test_decode_window_parity(B, T, Hk, Hv, Dk, Dv, commit, act):
    rng = np.random.default_rng(B * 100 + T * 10 + Dk + Dv + commit)
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    w = _window_tokens(rng, B, T, Hk, Hv, Dk, Dv, act)
    d = DT[act]
    dw = {n: to_dev(x, torch.float32 if n == "g" else d, DEV) for n, x in w.items()}
    s_in = to_dev(S0, torch.float32, DEV)
    s_out = torch.full_like(s_in, float("nan"))
    _, y = gdn.gdn_decode_window(s_in, s_out, dw["q"], dw["k"], dw["v"], dw["g"], dw["beta"], commit=commit)
    torch.cuda.synchronize()
    S_ref, y_ref = oracle.gdn_window(S0, w["q"], w["k"], w["v"], w["g"], w["beta"], commit=commit)
    if commit == 0:
        assert torch.isnan(s_out).all()          # a verify window writes no state
    else:
        assert maxrel(to_np(s_out), S_ref) <= 1e-5
    yv = to_np(y)
    if act == "f32":
        assert maxrel(yv, y_ref) <= 1e-5
    else:
        check_bf16_out(yv, y_ref, "window y")
    assert np.array_equal(to_np(s_in).astype(np.float32), S0)  # state_in untouched


def test_decode_window_matches_single_steps_and_runs_in_place():
    """A committed 4-token window equals four gdn_decode_step calls (up to
    rounding order) and gives the same result in place."""
    rng = np.random.default_rng(31)
    B, T, Hk, Hv, Dk, Dv = 4, 4, 2, 6, 128, 128
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    w = _window_tokens(rng, B, T, Hk, Hv, Dk, Dv, "bf16")
    dw = {n: to_dev(x, torch.float32 if n == "g" else torch.bfloat16, DEV) for n, x in w.items()}
    S, ys = to_dev(S0, torch.float32, DEV), []
    for t in range(T):
        S, yt = gdn.gdn_decode_step(S, None, dw["q"][:, t].contiguous(), dw["k"][:, t].contiguous(),
                                    dw["v"][:, t].contiguous(), dw["g"][:, t].contiguous(),
                                    dw["beta"][:, t].contiguous())
        ys.append(yt)
    y_steps = torch.stack(ys, dim=1)
    s_io = to_dev(S0, torch.float32, DEV)
    _, y_win = gdn.gdn_decode_window(s_io, s_io, dw["q"], dw["k"], dw["v"], dw["g"], dw["beta"])
    torch.cuda.synchronize()
    assert maxrel(to_np(s_io), to_np(S)) <= 1e-6
    assert maxrel(to_np(y_win), to_np(y_steps)) <= 1e-2  # bf16 outputs of near-identical fp32 values
    assert relF(to_np(y_win), to_np(y_steps)) <= 1e-3


def test_committed_window_equals_the_fixed_length_prefill():
    """A committed 8-token window is gdn_chunk_prefill_fixed with no norm and
    scale 1 on the same [B, T, H, D] layouts (the faster route for T >= 4)."""
    rng = np.random.default_rng(32)
    B, T, Hk, Hv, Dk, Dv = 6, 8, 2, 6, 128, 128
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    w = _window_tokens(rng, B, T, Hk, Hv, Dk, Dv, "bf16")
    dw = {n: to_dev(x, torch.float32 if n == "g" else torch.bfloat16, DEV) for n, x in w.items()}
    s_win = to_dev(S0, torch.float32, DEV)
    _, y_win = gdn.gdn_decode_window(s_win, s_win, dw["q"], dw["k"], dw["v"], dw["g"], dw["beta"])
    s_fix = to_dev(S0, torch.float32, DEV)
    y_fix = gdn.gdn_chunk_prefill_fixed(dw["q"], dw["k"], dw["v"], dw["g"], dw["beta"].float().contiguous(),
                                        s_fix, chunk=8, scale=1.0, l2norm=False)
    torch.cuda.synchronize()
    S_ref, y_ref = oracle.gdn_window(S0, w["q"], w["k"], w["v"], w["g"], w["beta"])
    assert maxrel(to_np(s_win), S_ref) <= 1e-5
    assert maxrel(to_np(s_fix), S_ref) <= 1e-3
    check_bf16_out(to_np(y_fix), y_ref, "fixed-length y")
    check_bf16_out(to_np(y_win), y_ref, "window y")


@pytest.mark.parametrize("B,T,chunk,act", [
    (6, 8, 8, "bf16"),     # 36 chunk-loop workgroups: the half-width kernel
    (6, 16, 8, "bf16"),    # two chunks per sequence
    (48, 8, 8, "bf16"),    # 288 workgroups, more than the CUs
    (4, 16, 16, "f32"),    # fp32 activations: the register-fragment kernel
])
def test_verify_window_on_the_chunked_path(B, T, chunk, act):
    """A verify window (nothing committed) is gdn_chunk_prefill_fixed with
    GDN_KEEP_STATE, no norm and scale 1: y as the oracle's verify window, the
    state bit for bit unchanged, and y bit for bit the y of the same call
    without the flag (which does commit)."""
    rng = np.random.default_rng(B * 10 + T + chunk)
    Hk, Hv, Dk, Dv = 2, 6, 128, 128
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    w = _window_tokens(rng, B, T, Hk, Hv, Dk, Dv, act)
    d = DT[act]
    dw = {n: to_dev(x, torch.float32 if n == "g" else d, DEV) for n, x in w.items()}
    beta32 = dw["beta"].float().contiguous()
    s_keep = to_dev(S0, torch.float32, DEV)
    y_keep = gdn.gdn_chunk_prefill_fixed(dw["q"], dw["k"], dw["v"], dw["g"], beta32, s_keep, chunk=chunk,
                                         scale=1.0, l2norm=False, keep_state=True)
    s_commit = to_dev(S0, torch.float32, DEV)
    y_commit = gdn.gdn_chunk_prefill_fixed(dw["q"], dw["k"], dw["v"], dw["g"], beta32, s_commit, chunk=chunk,
                                           scale=1.0, l2norm=False)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(s_keep).astype(np.float32), S0)
    assert torch.equal(y_keep, y_commit)
    _, y_ref = oracle.gdn_window(S0, w["q"], w["k"], w["v"], w["g"], w["beta"], commit=0)
    if act == "f32":
        assert maxrel(to_np(y_keep), y_ref) <= 1e-3
    else:
        check_bf16_out(to_np(y_keep), y_ref, "verify window y")
