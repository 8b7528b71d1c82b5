"""GPU parity of gdn_prefill_gates + gdn_chunk_prefill against the fp64
token-by-token oracle, and bit-exact handling of cu_seqlens/cache_indices.

Tolerances: pool state max relative error <= 1e-3; y max relative <= 1e-3
when fp32, and when bf16 element by element (tests.helpers.check_bf16_out:
relative Frobenius <= 2e-2, max |error| <= 1e-2 of the largest value, every
row's max |error| <= 2e-2 of that row's largest); index handling bit-exact.
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


def _warm_pool(rng, P, Hk, Hv, Dk, Dv, steps=synth.WARMUP_STEPS):
    """Pool slots warmed by `steps` oracle decode steps (decode-batch
    distributions), handed over as float32."""
    S = np.zeros((P, Hv, Dv, Dk))
    for _ in range(steps):
        S, _ = oracle_decode_batched(S, synth.decode_token(rng, P, Hk, Hv, Dk, Dv))
    return S.astype(np.float32)


def _run_gpu(inp, pool0, chunk, act, l2norm=True, scale=None):
    d = DT[act]
    a, b = to_dev(inp["a"], d, DEV), to_dev(inp["b"], d, DEV)
    g, beta = gdn.gdn_prefill_gates(a, b, to_dev(inp["A_log"], torch.float32, DEV),
                                    to_dev(inp["dt_bias"], torch.float32, DEV))
    pool = to_dev(pool0, torch.float32, DEV)
    T, Hv, Dv = inp["v"].shape
    y = torch.full((T, Hv, Dv), float("nan"), dtype=d, device=DEV)
    ci = to_dev(inp["cache_indices"], torch.int64, DEV)
    cu = to_dev(inp["cu_seqlens"], torch.int64, DEV)
    assert gdn.gdn_validate_varlen(cu, ci, T, pool0.shape[0]) == 0
    gdn.gdn_chunk_prefill(to_dev(inp["q"], d, DEV), to_dev(inp["k"], d, DEV), to_dev(inp["v"], d, DEV),
                          g, beta, pool, ci, cu, chunk=chunk, scale=scale, l2norm=l2norm, y=y)
    torch.cuda.synchronize()
    return pool, y


def _run_oracle(inp, pool0, l2norm=True, scale=None):
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    return oracle.gdn_prefill(inp["q"], inp["k"], inp["v"], g, beta, pool0, inp["cache_indices"],
                              inp["cu_seqlens"], scale=scale, l2norm=l2norm)


def _check(pool_gpu, y_gpu, P_ref, y_ref, pool0, inp, act):
    P = to_np(pool_gpu)
    assert maxrel(P, P_ref) <= 1e-3
    yv = to_np(y_gpu)
    assert not np.isnan(yv).any()
    if act == "f32":
        assert maxrel(yv, y_ref) <= 1e-3
    else:
        check_bf16_out(yv, y_ref, "y")
    used = set(int(s) for s in inp["cache_indices"])
    lens = np.diff(inp["cu_seqlens"])
    for s, slot in enumerate(inp["cache_indices"]):
        if lens[s] == 0:
            used.discard(int(slot))
    for slot in range(pool0.shape[0]):
        if slot not in used:
            assert np.array_equal(to_np(pool_gpu[slot]).astype(np.float32), pool0[slot]), slot


def test_tiny_fp32_decode_then_prefill():
    """Tiny fp32 workload: one decode step from zero at B=2, Hk=2, Hv=4,
    Dk=Dv=32, then one 16-token sequence (chunk 8) into the pool made of the
    two decoded states, writing slot 1; slot 0 must come out bit-identical."""
    c = synth.TINY
    rng = np.random.default_rng(0)
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv, act="f32")
    S_ref, y_ref = oracle.gdn_step(np.zeros((B, Hv, Dv, Dk)), tok["q"], tok["k"], tok["v"], tok["g"],
                                   tok["beta"])
    t = {n: to_dev(a, torch.float32, DEV) for n, a in tok.items()}
    S_gpu, y_gpu = gdn.gdn_decode_step(torch.zeros((B, Hv, Dv, Dk), device=DEV), None, t["q"], t["k"],
                                       t["v"], t["g"], t["beta"])
    assert maxrel(to_np(S_gpu), S_ref) <= 1e-5 and maxrel(to_np(y_gpu), y_ref) <= 1e-5
    pool0 = S_ref.astype(np.float32)
    inp = synth.prefill_inputs(rng, [c["prefill_len"]], Hk, Hv, Dk, Dv, pool_size=B, act="f32")
    inp["cache_indices"] = np.array([1], dtype=np.int64)
    pool, y = _run_gpu(inp, pool0, c["chunk"], "f32")
    P_ref, yr = _run_oracle(inp, pool0)
    _check(pool, y, P_ref, yr, pool0, inp, "f32")
    assert np.array_equal(to_np(pool[0]).astype(np.float32), pool0[0])


CASES = [
    # lengths, Hk, Hv, Dk, Dv, chunk, act
    ([1, 7, 64, 65, 130, 0, 200], 2, 4, 128, 128, 64, "bf16"),
    ([33, 64, 95, 1], 1, 3, 64, 96, 32, "bf16"),
    ([50, 17, 0, 31], 2, 2, 32, 64, 16, "bf16"),
    ([40, 9], 1, 2, 128, 32, 8, "bf16"),
    ([70, 3, 128], 2, 4, 128, 64, 64, "f32"),
    ([45, 16], 1, 1, 64, 32, 32, "f32"),
    ([100, 300], 1, 2, 128, 256, 64, "bf16"),      # two value blocks per head
    ([37, 100, 5], 2, 4, 128, 128, 32, "bf16"),    # 32-row tiles, eight waves
    ([90, 20], 1, 2, 64, 128, 64, "bf16"),         # Dk = 64 with eight waves
    ([77, 64], 1, 1, 32, 128, 16, "bf16"),         # Dk = 32, chunk 16, eight waves
    ([100, 37, 1, 0], 1, 2, 256, 128, 64, "bf16"), # Dk = 256: runs 32-token chunks
    ([70, 5, 33], 2, 4, 256, 64, 16, "bf16"),      # Dk = 256, four waves, chunk 16
    ([65, 40], 1, 1, 256, 96, 32, "bf16"),         # Dk = 256, two waves
    # key heads that are multiples of 32 but not powers of two
    ([100, 37, 0, 5], 2, 4, 96, 128, 64, "bf16"),  # Dk = 96, 64-token chunks
    ([70, 9], 1, 2, 96, 64, 16, "f32"),
    ([90, 33, 1], 1, 2, 160, 128, 64, "bf16"),     # Dk = 160: runs 32-token chunks
    ([64, 41], 2, 2, 192, 96, 32, "bf16"),
    ([77, 12], 1, 3, 224, 128, 64, "bf16"),
    # value heads per key head: 8, and 1
    ([66, 130], 1, 8, 128, 128, 64, "bf16"),
    ([129, 63], 4, 4, 128, 128, 64, "bf16"),
    ([20, 5, 64], 3, 6, 64, 64, 8, "f32"),         # fp32, chunk 8, three key heads
]


@pytest.mark.parametrize("lengths,Hk,Hv,Dk,Dv,chunk,act", CASES)
def test_prefill_parity(lengths, Hk, Hv, Dk, Dv, chunk, act):
    rng = np.random.default_rng(sum(lengths) + Dk + Dv + chunk)
    P = len(lengths) + 3
    pool0 = _warm_pool(rng, P, Hk, Hv, Dk, Dv, steps=4)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P, act=act)
    pool, y = _run_gpu(inp, pool0, chunk, act)
    P_ref, y_ref = _run_oracle(inp, pool0)
    _check(pool, y, P_ref, y_ref, pool0, inp, act)


def test_prefill_long_memory():
    """Slowly decaying heads (A_log = -7: log-gates of about -6e-4 per token)
    over 1900 tokens: the state carries information across all 30 chunks, so
    every chunk's state-side product must keep fp32-grade accuracy."""
    rng = np.random.default_rng(5)
    Hk, Hv, Dk, Dv = 1, 2, 128, 128
    pool0 = _warm_pool(rng, 3, Hk, Hv, Dk, Dv, steps=4)
    inp = synth.prefill_inputs(rng, [700, 1200], Hk, Hv, Dk, Dv, pool_size=3)
    inp["A_log"] = np.full(Hv, -7.0, dtype=np.float32)
    g, _ = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    assert g.sum(axis=0).max() > -2.0          # the memory really is long
    pool, y = _run_gpu(inp, pool0, 64, "bf16")
    P_ref, y_ref = _run_oracle(inp, pool0)
    _check(pool, y, P_ref, y_ref, pool0, inp, "bf16")


def test_prefill_long_memory_dk256():
    """The long-memory case at Dk = 256 (32-token chunks: 60 chunk steps over
    the longer sequence), where the state-side products span twice the width."""
    rng = np.random.default_rng(6)
    Hk, Hv, Dk, Dv = 1, 2, 256, 128
    pool0 = _warm_pool(rng, 3, Hk, Hv, Dk, Dv, steps=4)
    inp = synth.prefill_inputs(rng, [700, 1200], Hk, Hv, Dk, Dv, pool_size=3)
    inp["A_log"] = np.full(Hv, -7.0, dtype=np.float32)
    g, _ = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    assert g.sum(axis=0).max() > -2.0
    pool, y = _run_gpu(inp, pool0, 64, "bf16")
    P_ref, y_ref = _run_oracle(inp, pool0)
    _check(pool, y, P_ref, y_ref, pool0, inp, "bf16")


def test_prefill_without_l2norm_and_explicit_scale():
    rng = np.random.default_rng(21)
    Hk, Hv, Dk, Dv = 1, 2, 64, 64
    pool0 = _warm_pool(rng, 3, Hk, Hv, Dk, Dv, steps=2)
    inp = synth.prefill_inputs(rng, [37, 70], Hk, Hv, Dk, Dv, pool_size=3)
    # unit-norm keys so that the un-normalised recurrence stays bounded
    k = inp["k"].astype(np.float64)
    inp["k"] = synth.round_bf16((k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32))
    pool, y = _run_gpu(inp, pool0, 64, "bf16", l2norm=False, scale=0.3)
    P_ref, y_ref = _run_oracle(inp, pool0, l2norm=False, scale=0.3)
    _check(pool, y, P_ref, y_ref, pool0, inp, "bf16")


def _gpu_prefill_seq(inp, pool_dev, chunk, sel, act="bf16"):
    """Run a subset of sequences `sel` (in that order) packed together."""
    d = DT[act]
    cu = inp["cu_seqlens"]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in sel]).astype(np.int64)
    lens = [int(cu[s + 1] - cu[s]) for s in sel]
    g, beta = gdn.gdn_prefill_gates(to_dev(inp["a"][idx], d, DEV), to_dev(inp["b"][idx], d, DEV),
                                    to_dev(inp["A_log"], torch.float32, DEV),
                                    to_dev(inp["dt_bias"], torch.float32, DEV))
    y = gdn.gdn_chunk_prefill(to_dev(inp["q"][idx], d, DEV), to_dev(inp["k"][idx], d, DEV),
                              to_dev(inp["v"][idx], d, DEV), g, beta, pool_dev,
                              to_dev(inp["cache_indices"][list(sel)], torch.int64, DEV),
                              to_dev(synth.cu_from_lengths(lens), torch.int64, DEV), chunk=chunk)
    return y, idx


def test_packing_order_and_repeat_are_bitwise_invariant():
    rng = np.random.default_rng(22)
    Hk, Hv, Dk, Dv = 2, 4, 128, 128
    lengths = [100, 0, 64, 3, 150]
    pool0 = _warm_pool(rng, 7, Hk, Hv, Dk, Dv, steps=2)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=7)
    pa = to_dev(pool0, torch.float32, DEV)
    ya, ia = _gpu_prefill_seq(inp, pa, 64, [0, 1, 2, 3, 4])
    pb = to_dev(pool0, torch.float32, DEV)
    yb, ib = _gpu_prefill_seq(inp, pb, 64, [4, 3, 2, 1, 0])
    pc = to_dev(pool0, torch.float32, DEV)
    yc, ic = _gpu_prefill_seq(inp, pc, 64, [0, 1, 2, 3, 4])
    assert torch.equal(pa, pb) and torch.equal(pa, pc)
    assert torch.equal(ya, yc)
    # same tokens, different packed positions: compare per token
    pos_b = {int(t): i for i, t in enumerate(ib)}
    perm = torch.tensor([pos_b[int(t)] for t in ia], device=DEV)
    assert torch.equal(ya, yb[perm])


def test_chunk_aligned_resume_is_bitwise_equal():
    rng = np.random.default_rng(23)
    Hk, Hv, Dk, Dv = 2, 2, 128, 64
    pool0 = _warm_pool(rng, 2, Hk, Hv, Dk, Dv, steps=2)
    inp = synth.prefill_inputs(rng, [192], Hk, Hv, Dk, Dv, pool_size=2)
    whole = to_dev(pool0, torch.float32, DEV)
    y_all, _ = _gpu_prefill_seq(inp, whole, 64, [0])
    split = synth.prefill_inputs(np.random.default_rng(0), [128, 64], Hk, Hv, Dk, Dv, pool_size=2)
    for n in ("q", "k", "v", "a", "b"):
        split[n] = inp[n]
    split["A_log"], split["dt_bias"] = inp["A_log"], inp["dt_bias"]
    slot = inp["cache_indices"][0]
    split["cache_indices"] = np.array([slot, slot], dtype=np.int64)
    part = to_dev(pool0, torch.float32, DEV)
    y1, _ = _gpu_prefill_seq(split, part, 64, [0])
    y2, _ = _gpu_prefill_seq(split, part, 64, [1])
    assert torch.equal(whole, part)
    assert torch.equal(y_all, torch.cat([y1, y2]))


def test_decode_loop_matches_prefill():
    """T decode steps on normalised, pre-scaled q/k equal a T-token prefill."""
    rng = np.random.default_rng(24)
    Hk, Hv, Dk, Dv, T = 2, 4, 128, 128, 40
    pool0 = _warm_pool(rng, 1, Hk, Hv, Dk, Dv, steps=2)
    inp = synth.prefill_inputs(rng, [T], Hk, Hv, Dk, Dv, pool_size=1, act="f32")
    pool, y = _run_gpu(inp, pool0, 16, "f32")
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    nrm = lambda x: x / np.sqrt(np.sum(x.astype(np.float64) ** 2, -1, keepdims=True) + 1e-6)
    S = to_dev(pool0, torch.float32, DEV)
    for t in range(T):
        q = to_dev((nrm(inp["q"][t]) * Dk ** -0.5)[None].astype(np.float32), torch.float32, DEV)
        k = to_dev(nrm(inp["k"][t])[None].astype(np.float32), torch.float32, DEV)
        S, yd = gdn.gdn_decode_step(S, S, q, k, to_dev(inp["v"][t][None], torch.float32, DEV),
                                    to_dev(g[t][None].astype(np.float32), torch.float32, DEV),
                                    to_dev(beta[t][None].astype(np.float32), torch.float32, DEV))
        assert maxrel(to_np(yd[0]), to_np(y[t])) <= 1e-3, t
    assert maxrel(to_np(S), to_np(pool)) <= 1e-4


def test_varlen_prefill_workload_sampled():
    """Varlen prefill workload: 8 sequences of U[512, 4096] tokens, Hk=16,
    Hv=48, Dk=Dv=128, bf16, chunk 64, pool of 16 warmed slots, random
    cache_indices, run as the bench runs it (gdn_chunk_prefill_raw: the
    gates from raw a, b inside the call).  The whole batch runs on the GPU;
    the oracle checks 3 sequences on 6 value heads (key heads 0 and 15)."""
    c = synth.PREFILL_VARLEN
    rng = np.random.default_rng(0)
    Hk, Hv, Dk, Dv, P = c["Hk"], c["Hv"], c["Dk"], c["Dv"], c["pool"]
    lengths = synth.seq_lengths(rng, c["n_seq"], c["len_lo"], c["len_hi"])
    pool0 = _warm_pool(rng, P, Hk, Hv, Dk, Dv)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    bf = torch.bfloat16
    pool = to_dev(pool0, torch.float32, DEV)
    y = gdn.gdn_chunk_prefill_raw(*(to_dev(inp[n], bf, DEV) for n in ("q", "k", "v", "a", "b")),
                                  to_dev(inp["A_log"], torch.float32, DEV), to_dev(inp["dt_bias"], torch.float32, DEV),
                                  pool, to_dev(inp["cache_indices"], torch.int64, DEV),
                                  to_dev(inp["cu_seqlens"], torch.int64, DEV), chunk=c["chunk"])
    torch.cuda.synchronize()
    yv = to_np(y)
    assert not np.isnan(yv).any()
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    cu = inp["cu_seqlens"]
    for s in (0, int(np.argmax(lengths)), 7):
        idx = np.arange(cu[s], cu[s + 1])
        slot = int(inp["cache_indices"][s])
        for hk in (0, 15):
            hs = np.arange(hk * 3, hk * 3 + 3)
            P_ref, y_ref = oracle.gdn_prefill(
                inp["q"][idx][:, [hk]], inp["k"][idx][:, [hk]], inp["v"][idx][:, hs],
                g[idx][:, hs], beta[idx][:, hs], pool0[[slot]][:, hs], [0], [0, len(idx)])
            assert maxrel(to_np(pool[slot][hs]), P_ref[0]) <= 1e-3, (s, hk)
            check_bf16_out(yv[idx][:, hs], y_ref, f"y of sequence {s}, key head {hk}")
    untouched = sorted(set(range(P)) - set(int(x) for x in inp["cache_indices"]))
    for slot in untouched:
        assert np.array_equal(to_np(pool[slot]).astype(np.float32), pool0[slot])



def test_one_sequence_of_65536_tokens_sampled():
    """The longest chain the tests run: one sequence of 65,536 tokens (1,024
    chunks, one after another) between two short ones, at the varlen
    workload's heads (Hk=16, Hv=48, Dk=Dv=128, bf16, chunk 64), through
    gdn_chunk_prefill_raw.  The oracle checks, on key head 9 (value heads
    27..29), the long sequence's final state and every output row, and the
    300-token sequence; and the one-token sequence on every head.  The unused
    pool slot stays untouched."""
    c = synth.PREFILL_VARLEN
    rng = np.random.default_rng(65536)
    Hk, Hv, Dk, Dv, P = c["Hk"], c["Hv"], c["Dk"], c["Dv"], 4
    lengths = [300, 65536, 1]
    pool0 = _warm_pool(rng, P, Hk, Hv, Dk, Dv)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    bf = torch.bfloat16
    pool = to_dev(pool0, torch.float32, DEV)
    y = gdn.gdn_chunk_prefill_raw(*(to_dev(inp[n], bf, DEV) for n in ("q", "k", "v", "a", "b")),
                                  to_dev(inp["A_log"], torch.float32, DEV), to_dev(inp["dt_bias"], torch.float32, DEV),
                                  pool, to_dev(inp["cache_indices"], torch.int64, DEV),
                                  to_dev(inp["cu_seqlens"], torch.int64, DEV), chunk=c["chunk"])
    torch.cuda.synchronize()
    yv = to_np(y)
    assert not np.isnan(yv).any()
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    cu = inp["cu_seqlens"]
    hk = 9
    hs = np.arange(hk * 3, hk * 3 + 3)
    for s in (1, 0):
        idx = np.arange(cu[s], cu[s + 1])
        slot = int(inp["cache_indices"][s])
        P_ref, y_ref = oracle.gdn_prefill(
            inp["q"][idx][:, [hk]], inp["k"][idx][:, [hk]], inp["v"][idx][:, hs],
            g[idx][:, hs], beta[idx][:, hs], pool0[[slot]][:, hs], [0], [0, len(idx)])
        assert maxrel(to_np(pool[slot][hs]), P_ref[0]) <= 1e-3, s
        check_bf16_out(yv[idx][:, hs], y_ref, f"y of sequence {s}")
    # the one-token sequence on every head
    t = [int(cu[2])]
    one = int(inp["cache_indices"][2])
    P_ref, y_ref = oracle.gdn_prefill(inp["q"][t], inp["k"][t], inp["v"][t], g[t], beta[t], pool0[[one]], [0], [0, 1])
    assert maxrel(to_np(pool[one]), P_ref[0]) <= 1e-3
    check_bf16_out(yv[t], y_ref, "y of the one-token sequence")
    unused = sorted(set(range(P)) - set(int(x) for x in inp["cache_indices"]))
    assert len(unused) == 1
    assert np.array_equal(to_np(pool[unused[0]]).astype(np.float32), pool0[unused[0]])


GATED_CASES = [
    # lengths, Hk, Hv, Dk, Dv, chunk, act   (bf16 with Dv = 128: norm fused in the chunk loop)
    ([1, 64, 130, 0, 77], 2, 4, 128, 128, 64, "bf16"),
    ([90, 33], 1, 2, 64, 128, 32, "bf16"),
    ([70, 5], 1, 2, 128, 256, 64, "bf16"),     # two workgroups per head: separate norm kernel
    ([40, 9], 1, 2, 64, 64, 16, "bf16"),
    ([45, 16], 1, 1, 64, 32, 32, "f32"),
    ([60, 7], 1, 2, 256, 128, 64, "bf16"),     # Dk = 256, fused norm
    # more chunk-loop workgroups than CUs (288), with the fused norm
    ([150, 60, 40, 100, 30, 20], 16, 48, 128, 128, 64, "bf16"),
]


@pytest.mark.parametrize("lengths,Hk,Hv,Dk,Dv,chunk,act", GATED_CASES)
def test_gated_prefill_parity(lengths, Hk, Hv, Dk, Dv, chunk, act):
    """y of gdn_chunk_prefill_gated equals the oracle's prefill output put
    through the oracle's gated RMS norm; the pool is bitwise that of the
    ungated call."""
    rng = np.random.default_rng(7 * sum(lengths) + Dv)
    P = len(lengths) + 2
    pool0 = _warm_pool(rng, P, Hk, Hv, Dk, Dv, steps=4)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P, act=act)
    T = int(sum(lengths))
    d = DT[act]
    z = torch.from_numpy(rng.standard_normal((T, Hv, Dv)).astype(np.float32)).to(d)
    gam = torch.from_numpy((1.0 + 0.2 * rng.standard_normal(Dv)).astype(np.float32))
    pool_plain, _ = _run_gpu(inp, pool0, chunk, act)
    a, b = to_dev(inp["a"], d, DEV), to_dev(inp["b"], d, DEV)
    g, beta = gdn.gdn_prefill_gates(a, b, to_dev(inp["A_log"], torch.float32, DEV),
                                    to_dev(inp["dt_bias"], torch.float32, DEV))
    pool = to_dev(pool0, torch.float32, DEV)
    y = torch.full((T, Hv, Dv), float("nan"), dtype=d, device=DEV)
    gdn.gdn_chunk_prefill(to_dev(inp["q"], d, DEV), to_dev(inp["k"], d, DEV), to_dev(inp["v"], d, DEV),
                          g, beta, pool, to_dev(inp["cache_indices"], torch.int64, DEV),
                          to_dev(inp["cu_seqlens"], torch.int64, DEV), chunk=chunk, y=y,
                          z=z.to(DEV), gamma=gam.to(DEV), eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool_plain)
    P_ref, o_ref = _run_oracle(inp, pool0)
    y_ref = oracle.gated_rmsnorm(o_ref, z.to(torch.float32).numpy(), gam.numpy(), eps=1e-6)
    yv = to_np(y)
    assert not np.isnan(yv).any()
    if act == "f32":
        assert maxrel(yv, y_ref) <= 1e-3
    else:
        check_bf16_out(yv, y_ref, "gated y")


FIXED_CASES = [
    # B, T, Hk, Hv, Dk, Dv, chunk, act
    (3, 100, 2, 4, 128, 128, 64, "bf16"),
    (2, 1, 1, 2, 64, 64, 32, "bf16"),
    (4, 77, 1, 3, 256, 128, 64, "bf16"),
    (2, 50, 1, 2, 64, 32, 16, "f32"),
    # one chunk per sequence and at least one workgroup per CU: the
    # single-operand-set chunk loop (bitwise the varlen call all the same)
    (64, 5, 2, 4, 128, 128, 8, "bf16"),
    (64, 16, 1, 4, 256, 128, 16, "bf16"),
    (64, 32, 2, 4, 64, 128, 32, "bf16"),
    (64, 7, 1, 4, 32, 128, 8, "bf16"),
    # more sequences than one wave maps (the varlen call runs a chunk-map
    # kernel; the fixed-length call finds every chunk's sequence by division)
    (100, 9, 2, 4, 64, 64, 8, "bf16"),
    (96, 8, 1, 4, 128, 128, 8, "bf16"),
    (300, 3, 1, 2, 256, 128, 16, "bf16"),
]


@pytest.mark.parametrize("B,T,Hk,Hv,Dk,Dv,chunk,act", FIXED_CASES)
def test_fixed_length_prefill(B, T, Hk, Hv, Dk, Dv, chunk, act):
    """gdn_chunk_prefill_fixed on [B, T, H, D] inputs and a [B, Hv, Dv, Dk]
    state equals the oracle with cu_seqlens = {0, T, ..., BT} and
    cache_indices = {0..B-1}, and is bitwise the varlen call on the same data."""
    rng = np.random.default_rng(B * 1000 + T + Dk + chunk)
    state0 = _warm_pool(rng, B, Hk, Hv, Dk, Dv, steps=4)
    inp = synth.prefill_inputs(rng, [T] * B, Hk, Hv, Dk, Dv, pool_size=B, act=act)
    inp["cache_indices"] = np.arange(B, dtype=np.int64)
    d = DT[act]
    g, beta = gdn.gdn_prefill_gates(to_dev(inp["a"], d, DEV), to_dev(inp["b"], d, DEV),
                                    to_dev(inp["A_log"], torch.float32, DEV),
                                    to_dev(inp["dt_bias"], torch.float32, DEV))
    q, k, v = (to_dev(inp[n], d, DEV) for n in ("q", "k", "v"))
    state = to_dev(state0, torch.float32, DEV)
    y = gdn.gdn_chunk_prefill_fixed(q.view(B, T, Hk, Dk), k.view(B, T, Hk, Dk), v.view(B, T, Hv, Dv),
                                    g.view(B, T, Hv), beta.view(B, T, Hv), state, chunk=chunk)
    torch.cuda.synchronize()
    P_ref, y_ref = _run_oracle(inp, state0)
    assert maxrel(to_np(state), P_ref) <= 1e-3
    if act == "f32":
        assert maxrel(to_np(y).reshape(B * T, Hv, Dv), y_ref) <= 1e-3
    else:
        check_bf16_out(to_np(y).reshape(B * T, Hv, Dv), y_ref, "fixed-length y")
    pool = to_dev(state0, torch.float32, DEV)
    y2 = gdn.gdn_chunk_prefill(q, k, v, g, beta, pool, to_dev(inp["cache_indices"], torch.int64, DEV),
                               to_dev(inp["cu_seqlens"], torch.int64, DEV), chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(pool, state)
    assert torch.equal(y2.view(B, T, Hv, Dv), y)


@pytest.mark.parametrize("N", [2500, 5000])
def test_many_short_sequences(N):
    """2,500 or 5,000 sequences of 0..6 tokens (more sequences than the
    chunk-map scan has threads, so each thread scans a range; past 4,096 the
    map reads counts and order back from memory instead of LDS): every
    sequence and slot matches the oracle, empty sequences leave their slots
    untouched."""
    rng = np.random.default_rng(77 + N)
    Hk, Hv, Dk, Dv = 1, 2, 32, 32
    lengths = rng.integers(0, 7, size=N)
    P = N + 5
    pool0 = (0.3 * rng.standard_normal((P, Hv, Dv, Dk))).astype(np.float32)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P, act="bf16")
    pool, y = _run_gpu(inp, pool0, 8, "bf16")
    P_ref, y_ref = _run_oracle(inp, pool0)
    _check(pool, y, P_ref, y_ref, pool0, inp, "bf16")


def test_a_few_hundred_sequences():
    """200 sequences of 0..40 tokens: mixed one- and multi-chunk sequences
    and more chunk-loop workgroups than CUs.  Every sequence and slot
    matches the oracle."""
    rng = np.random.default_rng(83)
    N, Hk, Hv, Dk, Dv = 200, 1, 2, 64, 128
    lengths = rng.integers(0, 41, size=N)
    P = N + 3
    pool0 = (0.3 * rng.standard_normal((P, Hv, Dv, Dk))).astype(np.float32)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P, act="bf16")
    pool, y = _run_gpu(inp, pool0, 16, "bf16")
    P_ref, y_ref = _run_oracle(inp, pool0)
    _check(pool, y, P_ref, y_ref, pool0, inp, "bf16")


def test_split_of_the_longest_sequence_only():
    """Four sequences at 48 value heads (192 chunk-loop workgroups): idle CUs
    leave room to run only the longest as two half-width workgroups per head;
    the others stay whole.  Checked on sampled heads of every sequence."""
    rng = np.random.default_rng(81)
    lengths, Hk, Hv, Dk, Dv, P = [1000, 130, 70, 40], 16, 48, 128, 128, 6
    pool0 = _warm_pool(rng, P, Hk, Hv, Dk, Dv, steps=2)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    pool, y = _run_gpu(inp, pool0, 64, "bf16")
    yv = to_np(y)
    assert not np.isnan(yv).any()
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    cu = inp["cu_seqlens"]
    for s in range(len(lengths)):
        idx = np.arange(cu[s], cu[s + 1])
        slot = int(inp["cache_indices"][s])
        for hk in (0, 15):
            hs = np.arange(hk * 3, hk * 3 + 3)
            P_ref, y_ref = oracle.gdn_prefill(
                inp["q"][idx][:, [hk]], inp["k"][idx][:, [hk]], inp["v"][idx][:, hs],
                g[idx][:, hs], beta[idx][:, hs], pool0[[slot]][:, hs], [0], [0, len(idx)])
            assert maxrel(to_np(pool[slot][hs]), P_ref[0]) <= 1e-3, (s, hk)
            check_bf16_out(yv[idx][:, hs], y_ref, f"y of sequence {s}, key head {hk}")


@pytest.mark.parametrize("lengths", [
    [1250, 130, 1980, 70],             # CUs to spare: the longest splits
    [1100, 1200, 128, 1000, 100, 90],  # a full machine: none splits
])
def test_split_choice(lengths):
    """At 48 value heads.  Four sequences (192 chunk-loop workgroups, room
    for one split): the longest (31 chunks) is the third of the batch and
    shares the bit length of its chunk count with the first (20 chunks); it
    must be the one that runs as two half-width workgroups per head (the
    first, split instead, would leave the longest whole and the split
    refused).  Six sequences (288 workgroups, more than the CUs): all stay
    whole; the 1000-token sequence has a row of y where the state-side and
    in-chunk terms nearly cancel.  Checked on sampled heads of every
    sequence."""
    rng = np.random.default_rng(85)
    Hk, Hv, Dk, Dv, P = 16, 48, 128, 128, 8
    pool0 = _warm_pool(rng, P, Hk, Hv, Dk, Dv, steps=2)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    pool, y = _run_gpu(inp, pool0, 64, "bf16")
    yv = to_np(y)
    assert not np.isnan(yv).any()
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    cu = inp["cu_seqlens"]
    for s in range(len(lengths)):
        idx = np.arange(cu[s], cu[s + 1])
        slot = int(inp["cache_indices"][s])
        hk = (0, 15)[s % 2]
        hs = np.arange(hk * 3, hk * 3 + 3)
        P_ref, y_ref = oracle.gdn_prefill(
            inp["q"][idx][:, [hk]], inp["k"][idx][:, [hk]], inp["v"][idx][:, hs],
            g[idx][:, hs], beta[idx][:, hs], pool0[[slot]][:, hs], [0], [0, len(idx)])
        assert maxrel(to_np(pool[slot][hs]), P_ref[0]) <= 1e-3, (s, hk)
        check_bf16_out(yv[idx][:, hs], y_ref, f"y of sequence {s}, key head {hk}")


@pytest.mark.parametrize("Dk,keep", [(256, False), (96, True), (128, True)])
def test_raw_gates_wide_heads_and_keep_state(Dk, keep):
    """gdn_chunk_prefill_raw on other paths: Dk = 256 (32-token chunks) and
    Dk = 96, and with GDN_KEEP_STATE (the pool read only): y and the pool bit
    for bit those of gdn_prefill_gates + gdn_chunk_prefill with the same
    flags, y within the bf16 bounds of the oracle on one sequence."""
    rng = np.random.default_rng(96 + Dk)
    Hk, Hv, Dv, P = 2, 4, 64, 5
    lengths = [70, 0, 33, 129]
    pool0 = (0.3 * rng.standard_normal((P, Hv, Dv, Dk))).astype(np.float32)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    bf = torch.bfloat16
    q, k, v, a, b = (to_dev(inp[n], bf, DEV) for n in ("q", "k", "v", "a", "b"))
    A_log, dtb = to_dev(inp["A_log"], torch.float32, DEV), to_dev(inp["dt_bias"], torch.float32, DEV)
    ci = to_dev(inp["cache_indices"], torch.int64, DEV)
    cu = to_dev(inp["cu_seqlens"], torch.int64, DEV)
    pool_two = to_dev(pool0, torch.float32, DEV)
    g, beta = gdn.gdn_prefill_gates(a, b, A_log, dtb)
    y_two = gdn.gdn_chunk_prefill(q, k, v, g, beta, pool_two, ci, cu, chunk=64, keep_state=keep)
    pool_raw = to_dev(pool0, torch.float32, DEV)
    y_raw = gdn.gdn_chunk_prefill_raw(q, k, v, a, b, A_log, dtb, pool_raw, ci, cu, chunk=64, keep_state=keep)
    torch.cuda.synchronize()
    assert torch.equal(y_raw, y_two)
    assert torch.equal(pool_raw, pool_two)
    if keep:
        assert np.array_equal(to_np(pool_raw).astype(np.float32), pool0)
    s = 3
    idx = np.arange(inp["cu_seqlens"][s], inp["cu_seqlens"][s + 1])
    slot = int(inp["cache_indices"][s])
    g64, b64 = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    P_ref, y_ref = oracle.gdn_prefill(inp["q"][idx], inp["k"][idx], inp["v"][idx], g64[idx], b64[idx],
                                      pool0[[slot]], [0], [0, len(idx)])
    check_bf16_out(to_np(y_raw)[idx], y_ref, "raw y")
    if not keep:
        assert maxrel(to_np(pool_raw[slot]), P_ref[0]) <= 1e-3


@pytest.mark.parametrize("case", ["small-bf16", "small-f32", "workload", "many-bf16"])
def test_raw_gates_equal_the_two_calls(case):
    """gdn_chunk_prefill_raw (gates formed from a, b, A_log, dt_bias inside
    the call: in the WY pass for bf16, by the gates kernel into the
    workspace for fp32) equals gdn_prefill_gates + gdn_chunk_prefill bit for
    bit, y and pool, on a ragged batch, on the varlen workload, and on 300
    sequences (more than the WY launch maps itself: the chunk map then runs
    as a kernel of its own)."""
    rng = np.random.default_rng(95)
    if case == "workload":
        c = synth.PREFILL_VARLEN
        Hk, Hv, Dk, Dv, P, act = c["Hk"], c["Hv"], c["Dk"], c["Dv"], c["pool"], "bf16"
        lengths = synth.seq_lengths(rng, c["n_seq"], c["len_lo"], c["len_hi"])
    elif case == "many-bf16":
        Hk, Hv, Dk, Dv, P, act = 2, 4, 64, 64, 310, "bf16"
        lengths = rng.integers(0, 150, size=300)
    else:
        Hk, Hv, Dk, Dv, P, act = 2, 6, 64, 128, 7, case.split("-")[1]
        lengths = [100, 37, 0, 5, 64]
    pool0 = (0.3 * rng.standard_normal((P, Hv, Dv, Dk))).astype(np.float32)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P, act=act)
    d = DT[act]
    q, k, v, a, b = (to_dev(inp[n], d, DEV) for n in ("q", "k", "v", "a", "b"))
    A_log, dtb = to_dev(inp["A_log"], torch.float32, DEV), to_dev(inp["dt_bias"], torch.float32, DEV)
    ci = to_dev(inp["cache_indices"], torch.int64, DEV)
    cu = to_dev(inp["cu_seqlens"], torch.int64, DEV)
    pool_two = to_dev(pool0, torch.float32, DEV)
    g, beta = gdn.gdn_prefill_gates(a, b, A_log, dtb)
    y_two = gdn.gdn_chunk_prefill(q, k, v, g, beta, pool_two, ci, cu, chunk=64)
    pool_raw = to_dev(pool0, torch.float32, DEV)
    y_raw = gdn.gdn_chunk_prefill_raw(q, k, v, a, b, A_log, dtb, pool_raw, ci, cu, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(y_raw, y_two)
    assert torch.equal(pool_raw, pool_two)


@pytest.mark.parametrize("route", ["plain", "gated", "noalloc"])
def test_keep_state_reads_the_pool_only(route):
    """GDN_KEEP_STATE: the pool is bit for bit unchanged and y is bit for
    bit the y of the same call without the flag (plain varlen call on the
    half-width kernel, the fused gated norm, the allocation-free entry)."""
    rng = np.random.default_rng(90)
    lengths, Hk, Hv, Dk, Dv, P = [100, 37, 0, 5], 2, 4, 128, 128, 6
    pool0 = _warm_pool(rng, P, Hk, Hv, Dk, Dv, steps=2)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    bf = torch.bfloat16
    a, b = to_dev(inp["a"], bf, DEV), to_dev(inp["b"], bf, DEV)
    g, beta = gdn.gdn_prefill_gates(a, b, to_dev(inp["A_log"], torch.float32, DEV),
                                    to_dev(inp["dt_bias"], torch.float32, DEV))
    q, k, v = (to_dev(inp[n], bf, DEV) for n in ("q", "k", "v"))
    ci = to_dev(inp["cache_indices"], torch.int64, DEV)
    cu = to_dev(inp["cu_seqlens"], torch.int64, DEV)
    T = q.shape[0]
    extra = {}
    if route == "gated":
        extra = dict(z=to_dev(rng.standard_normal((T, Hv, Dv)).astype(np.float32), bf, DEV),
                     gamma=to_dev(rng.uniform(0.5, 1.5, Dv).astype(np.float32), torch.float32, DEV))

    def run(keep):
        pool = to_dev(pool0, torch.float32, DEV)
        if route == "noalloc":
            y = torch.empty((T, Hv, Dv), dtype=bf, device=DEV)
            gdn.gdn_chunk_prefill_noalloc(q, k, v, g, beta, pool, ci, cu, y, chunk=64, keep_state=keep)
        else:
            y = gdn.gdn_chunk_prefill(q, k, v, g, beta, pool, ci, cu, chunk=64, keep_state=keep, **extra)
        torch.cuda.synchronize()
        return pool, y

    pool_k, y_k = run(True)
    pool_c, y_c = run(False)
    assert np.array_equal(to_np(pool_k).astype(np.float32), pool0)
    assert torch.equal(y_k, y_c)
    assert not np.array_equal(to_np(pool_c).astype(np.float32), pool0)  # the call without it commits


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_batch_of_empty_sequences_leaves_the_pool_untouched(act):
    """Three sequences of zero tokens (T_tot = 0): every launch runs and finds
    no chunk; the pool, gated path included, is bitwise unchanged."""
    d = DT[act]
    rng = np.random.default_rng(91)
    Hk, Hv, Dk, Dv, P = 2, 4, 128, 128, 5
    pool0 = (0.3 * rng.standard_normal((P, Hv, Dv, Dk))).astype(np.float32)
    pool = to_dev(pool0, torch.float32, DEV)
    ci = torch.tensor([2, 0, 4], dtype=torch.int64, device=DEV)
    cu = torch.zeros(4, dtype=torch.int64, device=DEV)
    e = lambda *s, dt=d: torch.empty(s, dtype=dt, device=DEV)
    y = e(0, Hv, Dv)
    gdn.gdn_chunk_prefill(e(0, Hk, Dk), e(0, Hk, Dk), e(0, Hv, Dv), e(0, Hv, dt=torch.float32),
                          e(0, Hv, dt=torch.float32), pool, ci, cu, chunk=64, y=y)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(pool).astype(np.float32), pool0)
