"""gdn_chunk_prefill_noalloc (the library's static device workspace) against
gdn_chunk_prefill with a caller workspace, through the C ABI: two calls in a
row, the second with a smaller input, so the second runs over the first's
leftovers in the shared scratch.  Both entry points run the same kernels on
the same workspace layout, so pool and y must be bitwise equal; the smaller
call is also checked against the fp64 oracle at the prefill tolerances."""
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


def _inputs(rng, lengths, Hk, Hv, Dk, Dv, act):
    P = len(lengths) + 2
    pool0 = (0.3 * rng.standard_normal((P, Hv, Dv, Dk))).astype(np.float32)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P, act=act)
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    d = DT[act]
    dev = {n: to_dev(inp[n], d, DEV) for n in ("q", "k", "v")}
    dev["g"] = to_dev(g.astype(np.float32), torch.float32, DEV)
    dev["beta"] = to_dev(beta.astype(np.float32), torch.float32, DEV)
    dev["ci"] = to_dev(inp["cache_indices"], torch.int64, DEV)
    dev["cu"] = to_dev(inp["cu_seqlens"], torch.int64, DEV)
    return inp, g, beta, pool0, dev


def _both(dev, pool0, chunk):
    T, Hv, Dv = dev["v"].shape
    act = dev["v"].dtype
    pool_ws = to_dev(pool0, torch.float32, DEV)
    pool_na = to_dev(pool0, torch.float32, DEV)
    y_ws = torch.full((T, Hv, Dv), float("nan"), dtype=act, device=DEV)
    y_na = torch.full((T, Hv, Dv), float("nan"), dtype=act, device=DEV)
    args = (dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"])
    gdn.gdn_chunk_prefill(*args, pool_ws, dev["ci"], dev["cu"], chunk=chunk, y=y_ws)
    gdn.gdn_chunk_prefill_noalloc(*args, pool_na, dev["ci"], dev["cu"], y_na, chunk=chunk)
    torch.cuda.synchronize()
    return pool_ws, y_ws, pool_na, y_na


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_noalloc_equals_workspace_call_twice(act):
    rng = np.random.default_rng(2024 if act == "bf16" else 2025)
    Hk, Hv, Dk, Dv = 2, 6, 128, 128
    # first call: about 2,900 tokens over 7 sequences (ragged tails, an empty one)
    big = [1000, 640, 513, 0, 77, 300, 390] if act == "bf16" else [700, 300, 129]
    inp, g, beta, pool0, dev = _inputs(rng, big, Hk, Hv, Dk, Dv, act)
    need = gdn.gdn_chunk_prefill_workspace(int(sum(big)), len(big), Hk, Hv, Dk, Dv, 64, dev["v"].dtype)
    assert 0 < need <= 128 << 20
    p_ws, y_ws, p_na, y_na = _both(dev, pool0, 64)
    assert torch.equal(p_ws, p_na)
    assert torch.equal(y_ws, y_na)
    assert not torch.isnan(y_na.float()).any()
    # second call, smaller: the scratch still holds the first call's planes
    small = [150, 33, 64] if act == "bf16" else [90, 17]
    inp, g, beta, pool0, dev = _inputs(rng, small, Hk, Hv, Dk, Dv, act)
    p_ws, y_ws, p_na, y_na = _both(dev, pool0, 64)
    assert torch.equal(p_ws, p_na)
    assert torch.equal(y_ws, y_na)
    P_ref, y_ref = oracle.gdn_prefill(inp["q"], inp["k"], inp["v"], g, beta, pool0, inp["cache_indices"],
                                      inp["cu_seqlens"])
    assert maxrel(to_np(p_na), P_ref) <= 1e-3
    if act == "f32":
        assert maxrel(to_np(y_na), y_ref) <= 1e-3
    else:
        check_bf16_out(to_np(y_na), y_ref, "no-alloc y")


def test_noalloc_refuses_a_workspace_beyond_its_scratch():
    """A call that would need more than the 128 MiB scratch fails with
    GDN_ERR_WORKSPACE and leaves the pool untouched."""
    Hk, Hv, Dk, Dv, T = 16, 48, 128, 128, 20000
    assert gdn.gdn_chunk_prefill_workspace(T, 1, Hk, Hv, Dk, Dv, 64) > 128 << 20
    bf = torch.bfloat16
    q = torch.zeros((T, Hk, Dk), dtype=bf, device=DEV)
    v = torch.zeros((T, Hv, Dv), dtype=bf, device=DEV)
    gb = torch.zeros((T, Hv), dtype=torch.float32, device=DEV)
    pool = torch.ones((1, Hv, Dv, Dk), dtype=torch.float32, device=DEV)
    ci = torch.zeros(1, dtype=torch.int64, device=DEV)
    cu = torch.tensor([0, T], dtype=torch.int64, device=DEV)
    y = torch.empty((T, Hv, Dv), dtype=bf, device=DEV)
    with pytest.raises(gdn.GdnError) as err:
        gdn.gdn_chunk_prefill_noalloc(q, q, v, gb, gb, pool, ci, cu, y)
    assert err.value.status == -6
    torch.cuda.synchronize()
    assert bool((pool == 1).all())
