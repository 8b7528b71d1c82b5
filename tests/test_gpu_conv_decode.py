"""GPU parity of gdn_conv_decode_step (conv + SiLU, q/k norm, gates and the
decode step in one kernel) against the fp64 oracle chain: oracle.conv_silu
(one token per sequence, slot b = sequence b), oracle.gates, then
oracle.gdn_prefill with one token per sequence (which applies the q/k norm
and the query scale before the pinned decode step).

Tolerances: the decode step's (state max relative error <= 1e-5; y <= 1e-5
when fp32, element-wise bf16 bounds when bf16); the conv history, updated
in place, holds copies of inputs and must be bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import gated_deltanet_linear_gdn_amd as gdn
from gated_deltanet_linear_gdn_amd import synth
from tests.helpers import check_bf16_out, maxrel, to_dev, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _inputs(rng, B, Hk, Hv, Dk, Dv, act):
    """synth.layer_decode_inputs under the names used here (float32, widened
    exactly by the oracle)."""
    d = synth.layer_decode_inputs(rng, B, Hk, Hv, Dk, Dv, act=act)
    return dict(x=d["qkv"], W=d["conv_w"], hist=d["conv_state"], a=d["a"], b=d["b"], A_log=d["A_log"],
                dt_bias=d["dt_bias"])


def _oracle(S, inp, Hk, Hv, Dk, Dv, scale=None, l2norm=True):
    B = inp["x"].shape[0]
    ci, cu = np.arange(B, dtype=np.int64), np.arange(B + 1, dtype=np.int64)
    out, hist_new = oracle.conv_silu(inp["x"], inp["W"], inp["hist"], ci, cu)
    q = out[:, :Hk * Dk].reshape(B, Hk, Dk)
    k = out[:, Hk * Dk:2 * Hk * Dk].reshape(B, Hk, Dk)
    v = out[:, 2 * Hk * Dk:].reshape(B, Hv, Dv)
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    S_new, y = oracle.gdn_prefill(q, k, v, g, beta, S, ci, cu, scale=scale, l2norm=l2norm)
    return S_new, y, hist_new


def _gpu(S_dev, inp, Hk, act, out=None, scale=None, l2norm=True):
    """Returns (state_out, y, history after the call)."""
    d = DT[act]
    f32 = torch.float32
    hist = to_dev(inp["hist"], f32, DEV)
    S, y = gdn.gdn_conv_decode_step(S_dev, out, to_dev(inp["x"], d, DEV), to_dev(inp["W"], f32, DEV), hist,
                                    to_dev(inp["a"], d, DEV), to_dev(inp["b"], d, DEV),
                                    to_dev(inp["A_log"], f32, DEV), to_dev(inp["dt_bias"], f32, DEV), Hk,
                                    scale=scale, l2norm=l2norm)
    return S, y, hist


def _check(S_dev, y, hist_out, S_ref, y_ref, hist_ref, act):
    torch.cuda.synchronize()
    assert maxrel(to_np(S_dev), S_ref) <= 1e-5
    if act == "f32":
        assert maxrel(to_np(y), y_ref) <= 1e-5
    else:
        check_bf16_out(to_np(y), y_ref, "y")
    assert np.array_equal(to_np(hist_out), hist_ref)


SHAPES = [
    # B, Hk, Hv, Dk, Dv
    (3, 1, 3, 32, 32),
    (2, 2, 6, 64, 96),
    (3, 2, 4, 128, 128),
    (1, 1, 2, 128, 160),   # Dv not a multiple of the rows a workgroup covers
    (2, 3, 3, 256, 64),    # two q and two k channels per thread
    (5, 4, 8, 128, 32),
    (2, 1, 48, 32, 32),    # 48 value heads read one key head
    (2, 2, 4, 96, 64),     # head sizes that are not powers of two
    (2, 1, 2, 192, 128),
]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("B,Hk,Hv,Dk,Dv", SHAPES)
def test_conv_decode_parity(B, Hk, Hv, Dk, Dv, act):
    rng = np.random.default_rng(B * 1000 + Hk * 100 + Dk + Dv)
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    inp = _inputs(rng, B, Hk, Hv, Dk, Dv, act)
    S_dev, y, hist_out = _gpu(to_dev(S0, torch.float32, DEV), inp, Hk, act)
    _check(S_dev, y, hist_out, *_oracle(S0, inp, Hk, Hv, Dk, Dv), act)


def test_conv_decode_without_norm_and_explicit_scale_in_place():
    """flags 0 (no q/k norm) with an explicit scale, the state updated in
    place: equal to the oracle chain and, bitwise, to the functional call."""
    rng = np.random.default_rng(77)
    B, Hk, Hv, Dk, Dv = 3, 2, 4, 128, 64
    S0 = (0.3 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    inp = _inputs(rng, B, Hk, Hv, Dk, Dv, "bf16")
    S_f, y_f, h_f = _gpu(to_dev(S0, torch.float32, DEV), inp, Hk, "bf16", scale=0.3, l2norm=False)
    S_io = to_dev(S0, torch.float32, DEV)
    S_i, y_i, h_i = _gpu(S_io, inp, Hk, "bf16", out=S_io, scale=0.3, l2norm=False)
    torch.cuda.synchronize()
    assert S_i.data_ptr() == S_io.data_ptr()
    assert torch.equal(S_f, S_i) and torch.equal(y_f, y_i) and torch.equal(h_f, h_i)
    _check(S_i, y_i, h_i, *_oracle(S0, inp, Hk, Hv, Dk, Dv, scale=0.3, l2norm=False), "bf16")


def test_conv_decode_batch_b256_three_steps():
    """The large decode batch (B=256, Hk=16, Hv=48, Dk=Dv=128, bf16) as the
    bench runs it: states ping-pong between two buffers, the conv history is
    updated in place.  Step 1 is checked on the whole state, output and
    history; two more steps on 6 sampled sequences (the oracle follows their
    states and histories)."""
    c = synth.DECODE_B256
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    rng = np.random.default_rng(0)
    S0 = (0.1 * rng.standard_normal((B, Hv, Dv, Dk))).astype(np.float32)
    inp = _inputs(rng, B, Hk, Hv, Dk, Dv, "bf16")
    f32, bf = torch.float32, torch.bfloat16
    S = [to_dev(S0, f32, DEV), torch.empty((B, Hv, Dv, Dk), dtype=f32, device=DEV)]
    H = to_dev(inp["hist"], f32, DEV)
    W, A_log, dtb = (to_dev(inp[n], f32, DEV) for n in ("W", "A_log", "dt_bias"))
    ws = torch.empty(gdn.gdn_conv_decode_workspace(B, Hk, Hv, Dk, Dv), dtype=torch.uint8, device=DEV)
    sample = np.array([0, 3, 100, 171, 254, 255])
    S_ref, hist_ref = S0.astype(np.float64), inp["hist"]
    idx = torch.from_numpy(sample).to(DEV)
    for step in range(3):
        if step > 0:   # a new token (new raw channels and gate inputs), same weights
            new = _inputs(rng, B, Hk, Hv, Dk, Dv, "bf16")
            inp = dict(inp, x=new["x"], a=new["a"], b=new["b"])
        _, y = gdn.gdn_conv_decode_step(S[step % 2], S[(step + 1) % 2], to_dev(inp["x"], bf, DEV), W, H,
                                        to_dev(inp["a"], bf, DEV), to_dev(inp["b"], bf, DEV), A_log, dtb, Hk,
                                        workspace=ws)
        torch.cuda.synchronize()
        dst = (step + 1) % 2
        if step == 0:
            S_ref, y_ref, hist_ref = _oracle(S_ref, dict(inp, hist=hist_ref), Hk, Hv, Dk, Dv)
            _check(S[dst], y, H, S_ref, y_ref, hist_ref, "bf16")
            S_ref, hist_ref = S_ref[sample], hist_ref[sample]
            continue
        sub = {n: (inp[n][sample] if n in ("x", "a", "b") else inp[n]) for n in inp}
        S_ref, y_ref, hist_ref = _oracle(S_ref, dict(sub, hist=hist_ref), Hk, Hv, Dk, Dv)
        _check(S[dst][idx], y[idx], H[idx], S_ref, y_ref, hist_ref, "bf16")
