"""GPU parity of gdn_conv_prefill: the conv + SiLU prologue, the gates from
raw inputs, the chunked recurrence and (with z) the gated norm in one call.

Two references:
- the separate calls on the same device inputs (gdn_conv_silu, then
  gdn_chunk_prefill_raw, or gdn_prefill_gates + gdn_chunk_prefill with the
  norm): y, the state pool and the conv history must be the same bits;
- the fp64 oracle chain oracle.conv_silu -> oracle.gates ->
  oracle.gdn_prefill (-> oracle.gated_rmsnorm), with the convolved q, k, v
  rounded to bf16 in between (the activation dtype the recurrence reads):
  pool max relative error <= 1e-3, bf16 y relative Frobenius <= 2e-2 and
  max relative <= 1e-2, the history (copies of inputs) bit-exact, and every
  slot no non-empty sequence names untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_deltanet_linear_gdn_amd as gdn
from gated_deltanet_linear_gdn_amd import synth
from tests.helpers import check_bf16_out, maxrel, to_dev, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF = torch.bfloat16
F32 = torch.float32


def _case(rng, lengths, Hk, Hv, Dk, Dv, P):
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    T = int(inp["cu_seqlens"][-1])
    lay = synth.layer_inputs(rng, T, Hk, Hv, Dk, Dv, P)
    pool0 = (0.3 * rng.standard_normal((P, Hv, Dv, Dk))).astype(np.float32)
    return inp, lay, pool0


def _dev_inputs(inp, lay, pool0):
    d = {n: to_dev(inp[n], BF, DEV) for n in ("a", "b")}
    d.update({n: to_dev(inp[n], F32, DEV) for n in ("A_log", "dt_bias")})
    d.update({n: to_dev(inp[n], torch.int64, DEV) for n in ("cache_indices", "cu_seqlens")})
    d["qkv"] = to_dev(lay["qkv"], BF, DEV)
    d["conv_w"] = to_dev(lay["conv_w"], F32, DEV)
    d["z"] = to_dev(lay["z"], BF, DEV)
    d["gamma"] = to_dev(lay["gamma"], F32, DEV)
    d["hist"] = to_dev(lay["conv_state"], F32, DEV)
    d["pool"] = to_dev(pool0, F32, DEV)
    return d


def _fused(d, Hk, Hv, Dk, Dv, chunk, gated, keep=False):
    hist, pool = d["hist"].clone(), d["pool"].clone()
    y = gdn.gdn_conv_prefill(d["qkv"], d["conv_w"], hist, d["a"], d["b"], d["A_log"], d["dt_bias"], pool,
                             d["cache_indices"], d["cu_seqlens"], Hk, Hv, Dk, Dv, chunk=chunk,
                             keep_state=keep, z=d["z"] if gated else None, gamma=d["gamma"] if gated else None)
    torch.cuda.synchronize()
    return y, pool, hist


def _separate(d, Hk, Hv, Dk, Dv, chunk, gated):
    hist, pool = d["hist"].clone(), d["pool"].clone()
    ci, cu = d["cache_indices"], d["cu_seqlens"]
    q, k, v = gdn.gdn_conv_silu(d["qkv"], d["conv_w"], hist, ci, cu, Hk, Hv, Dk, Dv)
    if gated:
        g, beta = gdn.gdn_prefill_gates(d["a"], d["b"], d["A_log"], d["dt_bias"])
        y = gdn.gdn_chunk_prefill(q, k, v, g, beta, pool, ci, cu, chunk=chunk, z=d["z"], gamma=d["gamma"])
    else:
        y = gdn.gdn_chunk_prefill_raw(q, k, v, d["a"], d["b"], d["A_log"], d["dt_bias"], pool, ci, cu,
                                      chunk=chunk)
    torch.cuda.synchronize()
    return y, pool, hist


def _oracle(inp, lay, pool0, Hk, Hv, Dk, Dv, gated):
    ci, cu = inp["cache_indices"], inp["cu_seqlens"]
    out, href = oracle.conv_silu(lay["qkv"], lay["conv_w"], lay["conv_state"], ci, cu)
    out = synth.round_bf16(out).astype(np.float64)
    T = out.shape[0]
    nq = Hk * Dk
    q = out[:, :nq].reshape(T, Hk, Dk)
    k = out[:, nq:2 * nq].reshape(T, Hk, Dk)
    v = out[:, 2 * nq:].reshape(T, Hv, Dv)
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    P_ref, y_ref = oracle.gdn_prefill(q, k, v, g, beta, pool0, ci, cu)
    if gated:
        y_ref = oracle.gated_rmsnorm(y_ref, lay["z"], lay["gamma"])
    return y_ref, P_ref, href


CASES = [
    # lengths, Hk, Hv, Dk, Dv, chunk, gated
    ([5, 0, 1, 2, 3, 40], 2, 4, 32, 64, 8, False),       # empty, 1- and 2-token sequences (history mixing)
    ([130, 64, 7, 200], 2, 6, 64, 64, 16, True),
    ([300, 17, 4, 65], 1, 3, 128, 128, 64, True),        # the fused norm in the chunk loop
    ([300, 17, 4, 65], 1, 3, 128, 128, 64, False),
    ([257, 90], 2, 2, 96, 32, 32, False),                # key heads of 96
    ([100, 33], 1, 2, 256, 128, 64, True),               # Dk 256: 32-token chunks
    ([700, 1300, 2], 16, 48, 128, 128, 64, True),        # the layer's 10,240 channels
    ([37, 1, 0, 90, 3] * 14, 2, 16, 64, 32, 32, False),  # 70 sequences: the chunk map as its own kernel
    ([150, 66], 2, 2, 128, 128, 64, True),               # one value head per key head
    ([97, 12], 1, 8, 128, 64, 16, False),                # eight value heads per key head
    ([77, 20, 1], 1, 2, 128, 128, 64, False),            # exactly 64 channel groups per key head
]


@pytest.mark.parametrize("lengths,Hk,Hv,Dk,Dv,chunk,gated", CASES)
def test_conv_prefill_equals_separate_calls_and_oracle(lengths, Hk, Hv, Dk, Dv, chunk, gated):
    rng = np.random.default_rng(sum(lengths) + 7 * Hk + Dk + chunk)
    P = len(lengths) + 2
    print(f"conv_prefill lengths={lengths} Hk={Hk} Hv={Hv} Dk={Dk} Dv={Dv} chunk={chunk} gated={gated}",
          flush=True)
    inp, lay, pool0 = _case(rng, lengths, Hk, Hv, Dk, Dv, P)
    d = _dev_inputs(inp, lay, pool0)
    y2, pool2, hist2 = _fused(d, Hk, Hv, Dk, Dv, chunk, gated)
    y1, pool1, hist1 = _separate(d, Hk, Hv, Dk, Dv, chunk, gated)
    assert torch.equal(y2, y1)
    assert torch.equal(pool2, pool1)
    assert torch.equal(hist2, hist1)

    y_ref, P_ref, h_ref = _oracle(inp, lay, pool0, Hk, Hv, Dk, Dv, gated)
    yv = to_np(y2)
    assert not np.isnan(yv).any()
    check_bf16_out(yv, y_ref, "y")
    assert maxrel(to_np(pool2), P_ref) <= 1e-3
    np.testing.assert_array_equal(to_np(hist2).astype(np.float32), h_ref.astype(np.float32))
    named = {int(inp["cache_indices"][s]) for s in range(len(lengths)) if lengths[s] > 0}
    for slot in range(P):
        if slot not in named:
            assert torch.equal(pool2[slot], d["pool"][slot]), slot
            assert torch.equal(hist2[slot], d["hist"][slot]), slot


def test_conv_prefill_keep_state_leaves_pool_and_history():
    """GDN_KEEP_STATE: the same y bits, the pool and the conv history as they
    were (a verify pass over the prompt)."""
    rng = np.random.default_rng(3)
    lengths, Hk, Hv, Dk, Dv = [90, 2, 33], 2, 6, 128, 128
    P = 5
    inp, lay, pool0 = _case(rng, lengths, Hk, Hv, Dk, Dv, P)
    d = _dev_inputs(inp, lay, pool0)
    y_keep, pool_k, hist_k = _fused(d, Hk, Hv, Dk, Dv, 64, True, keep=True)
    y, _, _ = _fused(d, Hk, Hv, Dk, Dv, 64, True)
    assert torch.equal(y_keep, y)
    assert torch.equal(pool_k, d["pool"])
    assert torch.equal(hist_k, d["hist"])


def test_conv_prefill_chunks_continue_across_calls():
    """A sequence fed in two calls (the second resuming from the slot's state
    and conv history) equals the sequence in one call, within the oracle's
    bounds, and the history after both is the oracle's bit for bit."""
    rng = np.random.default_rng(11)
    Hk, Hv, Dk, Dv, P = 2, 4, 64, 64, 3
    L1, L2 = 70, 45
    inp, lay, pool0 = _case(rng, [L1 + L2], Hk, Hv, Dk, Dv, P)
    d = _dev_inputs(inp, lay, pool0)
    y_one, pool_one, hist_one = _fused(d, Hk, Hv, Dk, Dv, 16, False)
    # two calls over the same slot
    hist, pool = d["hist"].clone(), d["pool"].clone()
    ys = []
    for lo, hi in ((0, L1), (L1, L1 + L2)):
        cu = torch.tensor([0, hi - lo], dtype=torch.int64, device=DEV)
        ys.append(gdn.gdn_conv_prefill(d["qkv"][lo:hi].contiguous(), d["conv_w"], hist, d["a"][lo:hi].contiguous(),
                                       d["b"][lo:hi].contiguous(), d["A_log"], d["dt_bias"], pool,
                                       d["cache_indices"], cu, Hk, Hv, Dk, Dv, chunk=16))
    torch.cuda.synchronize()
    assert torch.equal(hist, hist_one)
    y_two = torch.cat(ys)
    y_ref, P_ref, h_ref = _oracle(inp, lay, pool0, Hk, Hv, Dk, Dv, False)
    check_bf16_out(to_np(y_two), y_ref, "y (two calls)")
    check_bf16_out(to_np(y_one), y_ref, "y (one call)")
    assert maxrel(to_np(pool), P_ref) <= 1e-3
    np.testing.assert_array_equal(to_np(hist).astype(np.float32), h_ref.astype(np.float32))


def test_conv_prefill_all_empty_is_a_no_op():
    rng = np.random.default_rng(4)
    Hk, Hv, Dk, Dv, P = 2, 4, 64, 64, 3
    inp, lay, pool0 = _case(rng, [0, 0], Hk, Hv, Dk, Dv, P)
    d = _dev_inputs(inp, lay, pool0)
    y, pool, hist = _fused(d, Hk, Hv, Dk, Dv, 64, False)
    assert y.shape[0] == 0
    assert torch.equal(pool, d["pool"])
    assert torch.equal(hist, d["hist"])


def test_conv_prefill_varlen_workload():
    """The bench's layer workload: 8 sequences of U[512, 4096] tokens,
    Hk=16, Hv=48, Dk=Dv=128 (10,240 raw channels), bf16, chunk 64, pool 16,
    with the gated norm.  Every output, slot and history entry equals the
    separate calls bit for bit; the history equals the oracle's; the oracle
    chain checks 2 sequences on key head 11 (value heads 33..35)."""
    c = synth.PREFILL_VARLEN
    rng = np.random.default_rng(0)
    Hk, Hv, Dk, Dv, P = c["Hk"], c["Hv"], c["Dk"], c["Dv"], c["pool"]
    lengths = synth.seq_lengths(rng, c["n_seq"], c["len_lo"], c["len_hi"])
    inp, lay, pool0 = _case(rng, lengths, Hk, Hv, Dk, Dv, P)
    d = _dev_inputs(inp, lay, pool0)
    y2, pool2, hist2 = _fused(d, Hk, Hv, Dk, Dv, c["chunk"], True)
    y1, pool1, hist1 = _separate(d, Hk, Hv, Dk, Dv, c["chunk"], True)
    assert torch.equal(y2, y1)
    assert torch.equal(pool2, pool1)
    assert torch.equal(hist2, hist1)
    ci, cu = inp["cache_indices"], inp["cu_seqlens"]
    out, h_ref = oracle.conv_silu(lay["qkv"], lay["conv_w"], lay["conv_state"], ci, cu)
    np.testing.assert_array_equal(to_np(hist2).astype(np.float32), h_ref.astype(np.float32))
    out = synth.round_bf16(out).astype(np.float64)
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    nq, hk, hs = Hk * Dk, 11, np.arange(33, 36)
    yv = to_np(y2)
    for s in (int(np.argmax(lengths)), 5):
        idx = np.arange(cu[s], cu[s + 1])
        slot = int(ci[s])
        o = out[idx]
        q = o[:, hk * Dk:(hk + 1) * Dk][:, None]
        k = o[:, nq + hk * Dk:nq + (hk + 1) * Dk][:, None]
        v = o[:, 2 * nq:].reshape(len(idx), Hv, Dv)[:, hs]
        P_ref, y_ref = oracle.gdn_prefill(q, k, v, g[idx][:, hs], beta[idx][:, hs], pool0[[slot]][:, hs], [0],
                                          [0, len(idx)])
        y_ref = oracle.gated_rmsnorm(y_ref, lay["z"][idx][:, hs], lay["gamma"])
        assert maxrel(to_np(pool2[slot][hs]), P_ref[0]) <= 1e-3, s
        check_bf16_out(yv[idx][:, hs], y_ref, f"y of sequence {s}, key head {hk}")
