"""GPU parity of the layer prologue (gdn_conv_silu) and epilogue
(gdn_gated_rmsnorm) against the fp64 oracle.

Tolerances: fp32 outputs max relative error <= 1e-5; bf16 outputs element
by element (tests.helpers.check_bf16_out: relative Frobenius <= 2e-2, max
relative <= 1e-2, per row <= 2e-2); the conv history (copies of
inputs) and every slot no sequence names bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_deltanet_linear_gdn_amd as gdn
from tests.helpers import check_bf16_out, maxrel, to_dev, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _round(x, act):
    """Host copy of what the device holds for activations of `act`."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16) if act == "bf16" else t).to(torch.float32).numpy().astype(np.float64)


def _conv_case(rng, lengths, Hk, Hv, Dk, Dv, P, act):
    C = 2 * Hk * Dk + Hv * Dv
    T = int(sum(lengths))
    x = _round(rng.standard_normal((T, C)), act)
    W = (0.5 * rng.standard_normal((C, 4))).astype(np.float32).astype(np.float64)
    hist = rng.standard_normal((P, C, 3)).astype(np.float32).astype(np.float64)
    ci = rng.permutation(P)[:len(lengths)].astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return x, W, hist, ci, cu


def _conv_gpu(x, W, hist, ci, cu, Hk, Hv, Dk, Dv, act):
    d = DT[act]
    h = to_dev(hist, torch.float32, DEV)
    q, k, v = gdn.gdn_conv_silu(to_dev(x, d, DEV), to_dev(W, torch.float32, DEV), h,
                                to_dev(ci, torch.int64, DEV), to_dev(cu, torch.int64, DEV), Hk, Hv, Dk, Dv)
    torch.cuda.synchronize()
    T = x.shape[0]
    out = np.concatenate([to_np(q).reshape(T, -1), to_np(k).reshape(T, -1), to_np(v).reshape(T, -1)], axis=1)
    return out, to_np(h)


def _check_out(out, ref, act):
    if act == "f32":
        assert maxrel(out, ref) <= 1e-5
    else:
        check_bf16_out(out, ref)


CONV_CASES = [
    # lengths, Hk, Hv, Dk, Dv, act
    ([5, 0, 1, 2, 3, 40], 2, 4, 32, 64, "f32"),
    ([5, 0, 1, 2, 3, 40], 2, 4, 32, 64, "bf16"),
    ([300, 17, 4], 1, 3, 64, 128, "bf16"),
    ([700, 1300], 16, 48, 128, 128, "bf16"),       # the layer's channel count, 2000 tokens
    ([260, 9], 16, 48, 128, 128, "f32"),
]


@pytest.mark.parametrize("lengths,Hk,Hv,Dk,Dv,act", CONV_CASES)
def test_conv_silu_parity(lengths, Hk, Hv, Dk, Dv, act):
    rng = np.random.default_rng(sum(lengths) + Hk + Dv)
    P = len(lengths) + 2
    x, W, hist, ci, cu = _conv_case(rng, lengths, Hk, Hv, Dk, Dv, P, act)
    out, h = _conv_gpu(x, W, hist, ci, cu, Hk, Hv, Dk, Dv, act)
    ref, href = oracle.conv_silu(x, W, hist, ci, cu)
    _check_out(out, ref, act)
    np.testing.assert_array_equal(h.astype(np.float32), href.astype(np.float32))
    named = {int(ci[s]) for s in range(len(lengths)) if lengths[s] > 0}
    for slot in range(P):
        if slot not in named:
            np.testing.assert_array_equal(h[slot].astype(np.float32), hist[slot].astype(np.float32))


def test_conv_silu_decode_steps_continue_a_prefill():
    """A prefill of ragged sequences, then three decode steps (one token per
    sequence) through the same history slots, equal the oracle run token by
    token over the concatenated inputs."""
    rng = np.random.default_rng(21)
    Hk, Hv, Dk, Dv, act = 2, 6, 64, 64, "bf16"
    lengths, P = [9, 2, 30], 5
    x, W, hist, ci, cu = _conv_case(rng, lengths, Hk, Hv, Dk, Dv, P, act)
    out, h = _conv_gpu(x, W, hist, ci, cu, Hk, Hv, Dk, Dv, act)
    ref, href = oracle.conv_silu(x, W, hist, ci, cu)
    _check_out(out, ref, act)
    B = len(lengths)
    for step in range(3):
        xd = _round(rng.standard_normal((B, x.shape[1])), act)
        cud = np.arange(B + 1, dtype=np.int64)
        out_d, h = _conv_gpu(xd, W, h, ci, cud, Hk, Hv, Dk, Dv, act)
        ref_d, href = oracle.conv_silu(xd, W, href, ci, cud)
        _check_out(out_d, ref_d, act)
        np.testing.assert_array_equal(h.astype(np.float32), href.astype(np.float32))


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("Dv", [32, 64, 128, 256])
def test_gated_rmsnorm_parity(Dv, act):
    rng = np.random.default_rng(Dv)
    T, Hv = 37, 5
    o = _round(2.0 * rng.standard_normal((T, Hv, Dv)), act)
    z = _round(rng.standard_normal((T, Hv, Dv)), act)
    gam = rng.standard_normal(Dv).astype(np.float32).astype(np.float64)
    o_d, z_d = to_dev(o, DT[act], DEV), to_dev(z, DT[act], DEV)
    g_d = to_dev(gam, torch.float32, DEV)
    y = gdn.gdn_gated_rmsnorm(o_d, z_d, g_d, eps=1e-6)
    ref = oracle.gated_rmsnorm(o, z, gam, eps=1e-6)
    _check_out(to_np(y), ref, act)
    # in place
    gdn.gdn_gated_rmsnorm(o_d, z_d, g_d, eps=1e-6, y=o_d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(o_d), to_np(y))


def test_gated_rmsnorm_layer_shape():
    """The layer's output shape: 2,000 tokens x 48 heads x 128, bf16."""
    rng = np.random.default_rng(5)
    T, Hv, Dv = 2000, 48, 128
    o = _round(rng.standard_normal((T, Hv, Dv)), "bf16")
    z = _round(rng.standard_normal((T, Hv, Dv)), "bf16")
    gam = (1.0 + 0.1 * rng.standard_normal(Dv)).astype(np.float32).astype(np.float64)
    y = gdn.gdn_gated_rmsnorm(to_dev(o, torch.bfloat16, DEV), to_dev(z, torch.bfloat16, DEV),
                              to_dev(gam, torch.float32, DEV))
    _check_out(to_np(y), oracle.gated_rmsnorm(o, z, gam), "bf16")
