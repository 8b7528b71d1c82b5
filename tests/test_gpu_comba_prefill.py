"""GPU parity of comba_chunk_prefill (the chunkwise Comba forward) against
the fp64 token-by-token oracle, through the C ABI.

Tolerances: pool state max relative error <= 1e-3; o (bf16) element by
element (tests.helpers.check_bf16_out: relative Frobenius <= 2e-2, max
|error| <= 1e-2 of the largest value, per row <= 2e-2 of the row's largest);
slots no sequence names bit-exact.
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
NAMES = ("q", "k", "v", "p", "beta", "g")


def _warm_pool(rng, P, H, K, V, steps=synth.WARMUP_STEPS):
    """Pool slots warmed by `steps` oracle Comba steps, as float32."""
    S = np.zeros((P, H, K, V))
    for _ in range(steps):
        t = synth.comba_token(rng, P, H, K, V)
        S, _ = oracle.comba_step(S, t["q"], t["k"], t["v"], t["p"], t["beta"], t["g"], inplace=True)
    return S.astype(np.float32)


def _dev_inputs(inp):
    return {n: to_dev(inp[n], torch.float32 if n == "g" else BF, DEV) for n in NAMES}


def _run_gpu(inp, pool0, chunk, scale=None):
    d = _dev_inputs(inp)
    pool = to_dev(pool0, torch.float32, DEV)
    T, H, V = inp["v"].shape
    o = torch.full((T, H, V), float("nan"), dtype=BF, device=DEV)
    ci = to_dev(inp["cache_indices"], torch.int64, DEV)
    cu = to_dev(inp["cu_seqlens"], torch.int64, DEV)
    assert gdn.gdn_validate_varlen(cu, ci, T, pool0.shape[0]) == 0
    gdn.comba_chunk_prefill(d["q"], d["k"], d["v"], d["p"], d["beta"], d["g"], pool, ci, cu, chunk=chunk,
                            scale=scale, o=o)
    torch.cuda.synchronize()
    return pool, o


def _check_untouched(pool, pool0, inp):
    lens = np.diff(inp["cu_seqlens"])
    used = {int(s) for s, n in zip(inp["cache_indices"], lens) if n > 0}
    for slot in range(pool0.shape[0]):
        if slot not in used:
            assert np.array_equal(to_np(pool[slot]).astype(np.float32), pool0[slot]), slot


CASES = [
    # lengths, H, K, V, chunk
    ([5, 0, 1, 70, 33], 2, 32, 32, 16),
    ([130, 64, 1], 2, 64, 64, 32),
    ([200, 77], 3, 128, 128, 64),
    ([150, 2], 2, 128, 256, 64),      # two workgroups per head
    ([100, 3], 1, 128, 96, 64),       # 32-column workgroups
    ([300, 129, 64], 2, 128, 128, 8),
    ([65, 31], 2, 64, 128, 64),
    ([90, 40, 1], 2, 256, 128, 64),   # K = 256: runs 32-token chunks
    ([100, 3], 2, 96, 128, 64),       # K = 96
    ([70, 35], 1, 192, 64, 32),       # K = 192: 32-token chunks
]


@pytest.mark.parametrize("lengths,H,K,V,chunk", CASES)
def test_comba_prefill_parity(lengths, H, K, V, chunk):
    rng = np.random.default_rng(sum(lengths) + K + V + chunk)
    P = len(lengths) + 2
    pool0 = _warm_pool(rng, P, H, K, V)
    inp = synth.comba_prefill_inputs(rng, lengths, H, K, V, P)
    pool, o = _run_gpu(inp, pool0, chunk)
    P_ref, o_ref = oracle.comba_prefill(*(inp[n] for n in NAMES), pool0, inp["cache_indices"],
                                        inp["cu_seqlens"])
    assert maxrel(to_np(pool), P_ref) <= 1e-3
    ov = to_np(o)
    assert not np.isnan(ov).any()
    check_bf16_out(ov, o_ref, "o")
    _check_untouched(pool, pool0, inp)


def test_comba_prefill_explicit_scale_and_chunk_independence():
    """An explicit query scale, and chunks of 16 and 64 tokens agree with each
    other to rounding (the chunk size is a schedule, not a semantics)."""
    rng = np.random.default_rng(71)
    lengths, H, K, V, P = [97, 40], 2, 128, 128, 3
    pool0 = _warm_pool(rng, P, H, K, V)
    inp = synth.comba_prefill_inputs(rng, lengths, H, K, V, P)
    P_ref, o_ref = oracle.comba_prefill(*(inp[n] for n in NAMES), pool0, inp["cache_indices"],
                                        inp["cu_seqlens"], scale=0.2)
    for chunk in (16, 64):
        pool, o = _run_gpu(inp, pool0, chunk, scale=0.2)
        assert maxrel(to_np(pool), P_ref) <= 1e-3, chunk
        check_bf16_out(to_np(o), o_ref, f"o at chunk {chunk}")


def test_comba_prefill_then_decode_steps():
    """A Comba prefill leaves each slot in the layout comba_decode_step reads:
    two decode steps over the prefilled slots continue the oracle's run."""
    rng = np.random.default_rng(72)
    lengths, H, K, V = [45, 130, 7], 2, 128, 128
    P = 3
    pool0 = _warm_pool(rng, P, H, K, V)
    inp = synth.comba_prefill_inputs(rng, lengths, H, K, V, P)
    inp["cache_indices"] = np.arange(P, dtype=np.int64)
    pool, _ = _run_gpu(inp, pool0, 64)
    P_ref, _ = oracle.comba_prefill(*(inp[n] for n in NAMES), pool0, inp["cache_indices"],
                                    inp["cu_seqlens"])
    S_dev, S_ref = pool, P_ref
    for _ in range(2):
        t = synth.comba_token(rng, P, H, K, V)
        d = {n: to_dev(t[n], torch.float32 if n == "g" else BF, DEV) for n in NAMES}
        S_dev, o = gdn.comba_decode_step(S_dev, None, d["q"], d["k"], d["v"], d["p"], d["beta"], d["g"])
        S_ref, o_ref = oracle.comba_step(S_ref, t["q"], t["k"], t["v"], t["p"], t["beta"], t["g"])
        torch.cuda.synchronize()
        assert maxrel(to_np(S_dev), S_ref) <= 1e-3
        check_bf16_out(to_np(o), o_ref, "decode o")


def test_comba_prefill_workload_sampled():
    """The Comba prefill workload: 8 sequences of U[512, 4096] tokens, H=32,
    K=V=128, bf16, chunk 64, pool of 16 warmed slots.  The whole batch runs on
    the GPU; the oracle follows 3 sequences on 2 heads each."""
    c = synth.COMBA_PREFILL_VARLEN
    rng = np.random.default_rng(0)
    H, K, V, P = c["H"], c["K"], c["V"], c["pool"]
    lengths = synth.seq_lengths(rng, c["n_seq"], c["len_lo"], c["len_hi"])
    pool0 = _warm_pool(rng, P, H, K, V)
    inp = synth.comba_prefill_inputs(rng, lengths, H, K, V, P)
    pool, o = _run_gpu(inp, pool0, c["chunk"])
    ov = to_np(o)
    assert not np.isnan(ov).any()
    cu = inp["cu_seqlens"]
    for s in (0, int(np.argmax(lengths)), 7):
        idx = np.arange(cu[s], cu[s + 1])
        slot = int(inp["cache_indices"][s])
        hs = [0, H - 1]
        P_ref, o_ref = oracle.comba_prefill(*(inp[n][idx][:, hs] for n in NAMES), pool0[[slot]][:, hs],
                                            [0], [0, len(idx)])
        assert maxrel(to_np(pool[slot][hs]), P_ref[0]) <= 1e-3, s
        check_bf16_out(ov[idx][:, hs], o_ref, f"o of sequence {s}")
    _check_untouched(pool, pool0, inp)


def test_comba_many_short_sequences():
    """2,500 sequences of 0..6 tokens over a pool of 2,505 slots."""
    rng = np.random.default_rng(78)
    N, H, K, V = 2500, 2, 32, 32
    lengths = rng.integers(0, 7, size=N)
    P = N + 5
    pool0 = (0.3 * rng.standard_normal((P, H, K, V))).astype(np.float32)
    inp = synth.comba_prefill_inputs(rng, lengths, H, K, V, P)
    pool, o = _run_gpu(inp, pool0, 16)
    P_ref, o_ref = oracle.comba_prefill(*(inp[n] for n in NAMES), pool0, inp["cache_indices"],
                                        inp["cu_seqlens"])
    assert maxrel(to_np(pool), P_ref) <= 1e-3
    check_bf16_out(to_np(o), o_ref, "o")
    _check_untouched(pool, pool0, inp)


def test_comba_prefill_long_memory():
    """Slowly decaying heads (log-gates of about -1e-3 per token) over 1,900
    tokens: the state carries information across all 30 chunks, so every
    chunk's state-side product must keep fp32-grade accuracy."""
    rng = np.random.default_rng(79)
    H, K, V, P = 2, 128, 128, 3
    pool0 = _warm_pool(rng, P, H, K, V)
    inp = synth.comba_prefill_inputs(rng, [700, 1200], H, K, V, P)
    inp["g"] = (-1e-3 * rng.random(inp["g"].shape)).astype(np.float32)
    assert inp["g"].sum(axis=0).min() > -2.0          # the memory really is long
    pool, o = _run_gpu(inp, pool0, 64)
    P_ref, o_ref = oracle.comba_prefill(*(inp[n] for n in NAMES), pool0, inp["cache_indices"],
                                        inp["cu_seqlens"])
    assert maxrel(to_np(pool), P_ref) <= 1e-3
    check_bf16_out(to_np(o), o_ref, "o")
    _check_untouched(pool, pool0, inp)


def test_comba_batch_of_empty_sequences_leaves_the_pool_untouched():
    """Two sequences of zero tokens (T_tot = 0): the pool is bitwise unchanged."""
    rng = np.random.default_rng(92)
    H, K, V, P = 2, 128, 128, 4
    pool0 = (0.3 * rng.standard_normal((P, H, K, V))).astype(np.float32)
    pool = to_dev(pool0, torch.float32, DEV)
    e = lambda *s, dt=BF: torch.empty(s, dtype=dt, device=DEV)
    ci = torch.tensor([3, 1], dtype=torch.int64, device=DEV)
    cu = torch.zeros(3, dtype=torch.int64, device=DEV)
    gdn.comba_chunk_prefill(e(0, H, K), e(0, H, K), e(0, H, V), e(0, H, K), e(0, H), e(0, H, dt=torch.float32),
                            pool, ci, cu, chunk=64, o=e(0, H, V))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(pool).astype(np.float32), pool0)
