#!/usr/bin/env python3
"""Throughput of the gated delta-rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Headline (``value``): ``gdn_decode_step`` on the large decode batch
B=256, Hk=16, Hv=48, Dk=Dv=128 (bf16 activations, fp32 state of 0.8 GB,
functional ping-pong state_in -> state_out), as achieved HBM GB/s over the
state bytes that must move each step (read once + written once).  A step is
one decode launch; K steps are timed with HIP events on the launch stream
after W untimed ones.  The same JSON line carries:
  * ``roofline``: that kernel's achieved GB/s against the 8 TB/s HBM peak;
  * ``comba``: ``comba_decode_step`` at B=128, H=32, K=V=128 (GB/s over the
    KBench canonical byte count);
  * ``prefill``: ``gdn_prefill_gates`` + ``gdn_chunk_prefill`` on 8 packed
    sequences of 512..4096 tokens (tokens/s and MFMA utilisation), when the
    library provides it;
  * ``torch_copy_GBps``: torch's own 2 GiB device-to-device copy (read +
    write bytes), for context: it runs below the decode kernel here;
  * ``cpu_baseline``: the fp64 CPU oracle on a bounded sample of the same
    decode workload, timed on this host's cores.
Inputs are seeded synthetic tensors (numpy PCG64, seed 0) resident in HBM
before timing starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published

# HBM bytes per B=256 decode launch from two rocprofv3 PMC runs of this bench
# (FETCH_SIZE x 2 + WRITE_SIZE x 1; the factors are what the same counters
# read for a 2 GiB device copy), valid for the kernel built from these
# sources only: after any change to them the figure is reported as null.
DECODE_TRAFFIC = {
    "bytes": 1659868570,
    "sources_sha256": {
        "gated_deltanet_linear_gdn_amd/csrc/gdn_decode.hip": "7736da6fa0045db52269febacb2aa07065fe5f09942bb1ce6155a50d9f207ccd",
        "gated_deltanet_linear_gdn_amd/csrc/gdn_decode_core.h": "a33da64879537627d6874f25c8cfee8a280d617ad4b467cc24edbd3161cb705b",
        "gated_deltanet_linear_gdn_amd/csrc/gdn_device.h": "01aacca146e67000b45bb4777947468b8e851857e2a3f9cd7869ecc457f9b6e7",
    },
}


def _decode_traffic():
    import hashlib
    for rel, want in DECODE_TRAFFIC["sources_sha256"].items():
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != want:
                return None
    return DECODE_TRAFFIC["bytes"]


def _dev(x, dtype, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dtype)


SETTLE_S = 0.2   # untimed running before each leg's warmup steps


def _timed(fn, steps, warmup):
    """Run fn(i) untimed for SETTLE_S seconds of wall time, then warmup
    times untimed, then `steps` times between HIP events recorded on the
    current stream (the stream the library launches on).  Returns seconds
    per step.

    The settle phase is there because a GPU that has been idle (host-side
    input generation between legs) runs its first launches slower: measured
    on MI355X, decode steps 10-35 after an idle second take 260-268 us
    against 251-255 us once settled, and a leg of 50 prefill calls started
    cold averaged 324 us against 286 us when run again right after.  It is
    timed by the wall clock, not by a call count estimated from the first
    call (which also loads the kernels' code)."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < SETTLE_S:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(warmup + i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def bench_decode(steps, warmup, device, B=None, Dk=None, inplace=False):
    """gdn_decode_step at the B=256 decode batch: functionally from state_in
    to state_out (ping-pong between two buffers), or with the state updated
    in place (state_out == state_in, as a serving loop keeps its state
    cache)."""
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    from gated_deltanet_linear_gdn_amd import synth
    c = synth.DECODE_B256
    B, Hk, Hv, Dk, Dv = B or c["B"], c["Hk"], c["Hv"], Dk or c["Dk"], c["Dv"]
    rng = np.random.default_rng(0)
    toks = []
    for _ in range(16):
        t = synth.decode_token(rng, B, Hk, Hv, Dk, Dv)
        toks.append({n: _dev(a, torch.float32 if n == "g" else torch.bfloat16, device)
                     for n, a in t.items()})
    bufs = [torch.zeros((B, Hv, Dv, Dk), dtype=torch.float32, device=device)]
    if not inplace:
        bufs.append(torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=device))
    y = torch.empty((B, Hv, Dv), dtype=torch.bfloat16, device=device)

    def step(i):
        t = toks[i % 16]
        src = bufs[0] if inplace else bufs[i % 2]
        dst = bufs[0] if inplace else bufs[(i + 1) % 2]
        gdn.gdn_decode_step(src, dst, t["q"], t["k"], t["v"], t["g"], t["beta"], y)

    for i in range(synth.WARMUP_STEPS):      # realistic state magnitudes, untimed
        step(i)
    sec = _timed(step, steps, warmup)
    state_bytes = 2 * B * Hv * Dv * Dk * 4
    act_bytes = B * (2 * Hk * Dk * 2 + Hv * Dv * 2 * 2 + Hv * (4 + 2))
    return dict(sec=sec, state_bytes=state_bytes, act_bytes=act_bytes,
                shape=dict(B=B, Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv))


def bench_window(steps, warmup, device, T, chunked=False, verify=False):
    """Decode windows of T tokens per sequence at the B=256 decode batch,
    committing all T (or, verify, none: every y, the state only read):
    gdn_decode_window (functional ping-pong, like the decode step) or,
    chunked, the same recurrence as gdn_chunk_prefill_fixed with no norm and
    scale 1 (in place, chunk = min(T, 64); GDN_KEEP_STATE to verify)."""
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    from gated_deltanet_linear_gdn_amd import synth
    c = synth.DECODE_B256
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    rng = np.random.default_rng(0)
    wins = []
    for _ in range(4):
        toks = [synth.decode_token(rng, B, Hk, Hv, Dk, Dv) for _ in range(T)]
        wins.append({n: _dev(np.stack([t[n] for t in toks], axis=1),
                             torch.float32 if n == "g" else torch.bfloat16, device) for n in toks[0]})
    bufs = [torch.zeros((B, Hv, Dv, Dk), dtype=torch.float32, device=device),
            torch.empty((B, Hv, Dv, Dk), dtype=torch.float32, device=device)]
    y = torch.empty((B, T, Hv, Dv), dtype=torch.bfloat16, device=device)
    chunk = min(max(T, 8), 64)
    ws = torch.empty(gdn.gdn_chunk_prefill_fixed_workspace(B, T, Hk, Hv, Dk, Dv, chunk) if chunked else 1,
                     dtype=torch.uint8, device=device)
    for w in wins:
        w["beta32"] = w["beta"].float().contiguous()

    def step(i):
        w = wins[i % 4]
        if chunked:
            gdn.gdn_chunk_prefill_fixed(w["q"], w["k"], w["v"], w["g"], w["beta32"], bufs[0], chunk=chunk,
                                        scale=1.0, l2norm=False, y=y, workspace=ws, keep_state=verify)
        else:
            gdn.gdn_decode_window(bufs[i % 2], bufs[(i + 1) % 2], w["q"], w["k"], w["v"], w["g"], w["beta"],
                                  y=y, commit=0 if verify else T)

    for i in range(4):
        step(i)
    sec = _timed(step, steps, warmup)
    return dict(sec=sec, tokens=B * T, state_bytes=(1 if verify else 2) * B * Hv * Dv * Dk * 4)


def bench_comba(steps, warmup, device):
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    from gated_deltanet_linear_gdn_amd import synth
    c = synth.COMBA_B128
    B, H, K, V = c["B"], c["H"], c["K"], c["V"]
    rng = np.random.default_rng(0)
    toks = []
    for _ in range(16):
        t = synth.comba_token(rng, B, H, K, V)
        toks.append({n: _dev(a, torch.float32 if n == "g" else torch.bfloat16, device)
                     for n, a in t.items()})
    bufs = [torch.zeros((B, H, K, V), dtype=torch.float32, device=device),
            torch.empty((B, H, K, V), dtype=torch.float32, device=device)]
    o = torch.empty((B, H, V), dtype=torch.bfloat16, device=device)

    def step(i):
        t = toks[i % 16]
        gdn.comba_decode_step(bufs[i % 2], bufs[(i + 1) % 2], t["q"], t["k"], t["v"], t["p"],
                              t["beta"], t["g"], o)

    for i in range(synth.WARMUP_STEPS):
        step(i)
    sec = _timed(step, steps, warmup)
    canonical = 2 * B * H * K * V * 4 + B * H * (6 * K + 4 * V + 6)
    return dict(sec=sec, bytes=canonical, shape=dict(B=B, H=H, K=K, V=V))


def prefill_flops_per_token(Hv, Dk, Dv, C):
    """Canonical FLOPs of the chunkwise prefill per token: per value head,
    the six C-wide contractions (K K^T, Q K^T, T K, T V, P V_new at 2C Dk or
    2C Dv each) and the three state contractions (W S_0, Q S_0, K^T V_new at
    2 Dk Dv each), counted as full products."""
    return Hv * (6 * Dk * Dv + C * (6 * Dk + 4 * Dv))


def prefill_issued_flops(lengths, Hk, Hv, Dk, Dv, C):
    """FLOPs the bf16 prefill kernels actually issue as MFMAs, hi/lo extra
    products included.  Chunk loop, per (chunk, value head) and per wave of 16
    value columns: X = K S and Y = Q S (S as hi + lo) take 4 (C/16)(Dk/32)
    16x16x32 products; Delta = (T diag beta) R takes 3 per lower 32-row block
    pair; P Delta one per pair; the state update 2 (Dk/16)(C/32).  WY pass, per
    (chunk, key head): the Gram blocks K K^T and Q K^T (2 (Dk/32) per lower
    16x16 block), and per value head 3 16x16x16 products per step of the
    blocked inverse.  Counts for C = 64 (the only tile the bench runs)."""
    assert C == 64
    MT, KB, DT, CKB = C // 16, Dk // 32, Dk // 16, C // 32
    pairs = sum(mt // 2 + 1 for mt in range(MT))
    per_wave = 4 * MT * KB + 3 * pairs + pairs + 2 * DT * CKB
    chunks = sum(-(-int(L) // C) for L in lengths)
    loop = chunks * Hv * (Dv // 16) * per_wave * 16 * 16 * 32 * 2
    npair = MT * (MT + 1) // 2
    inverse_steps = sum(d + 1 for d in range(1, MT) for _ in range(MT - d))  # mm3 calls
    wy = chunks * Hk * (npair * KB * 2 * 16 * 16 * 32 * 2
                        + (Hv // Hk) * inverse_steps * 3 * 16 * 16 * 16 * 2)
    return loop + wy


def prefill_min_bytes(T, n_seq, Hk, Hv, Dk, Dv, act_bytes=2):
    """Bytes a fused prefill must move: q, k, v, y and the raw gates a, b per
    token, and each sequence's state slot read and written once."""
    per_token = act_bytes * (2 * Hk * Dk + 2 * Hv * Dv + 2 * Hv)
    return T * per_token + n_seq * 2 * Hv * Dv * Dk * 4


def bench_prefill(steps, warmup, device, Dk=None, lengths=None, raw=True):
    """The varlen prefill from raw gate inputs: gdn_chunk_prefill_raw (the
    gates formed inside the WY pass), or with raw=False gdn_prefill_gates
    then gdn_chunk_prefill."""
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    from gated_deltanet_linear_gdn_amd import synth
    c = synth.PREFILL_VARLEN
    Hk, Hv, Dk, Dv, P, C = c["Hk"], c["Hv"], Dk or c["Dk"], c["Dv"], c["pool"], c["chunk"]
    rng = np.random.default_rng(0)
    drawn = synth.seq_lengths(rng, c["n_seq"], c["len_lo"], c["len_hi"])
    lengths = drawn if lengths is None else np.asarray(lengths, dtype=np.int64)
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    T = int(inp["cu_seqlens"][-1])
    bf = torch.bfloat16
    q, k, v = (_dev(inp[n], bf, device) for n in ("q", "k", "v"))
    a, b = _dev(inp["a"], bf, device), _dev(inp["b"], bf, device)
    A_log = _dev(inp["A_log"], torch.float32, device)
    dt_bias = _dev(inp["dt_bias"], torch.float32, device)
    ci = _dev(inp["cache_indices"], torch.int64, device)
    cu = _dev(inp["cu_seqlens"], torch.int64, device)
    # pool slots warmed like decode states: 16 decode steps from zero
    pool = torch.zeros((P, Hv, Dv, Dk), dtype=torch.float32, device=device)
    for _ in range(synth.WARMUP_STEPS):
        t = synth.decode_token(rng, P, Hk, Hv, Dk, Dv)
        td = {n: _dev(x, torch.float32 if n == "g" else bf, device) for n, x in t.items()}
        gdn.gdn_decode_step(pool, pool, td["q"], td["k"], td["v"], td["g"], td["beta"])
    g = torch.empty((T, Hv), dtype=torch.float32, device=device)
    beta = torch.empty_like(g)
    y = torch.empty((T, Hv, Dv), dtype=bf, device=device)
    wsf = gdn.gdn_chunk_prefill_raw_workspace if raw else gdn.gdn_chunk_prefill_workspace
    ws = torch.empty(wsf(T, len(lengths), Hk, Hv, Dk, Dv, C), dtype=torch.uint8, device=device)

    def step(i):
        if raw:
            gdn.gdn_chunk_prefill_raw(q, k, v, a, b, A_log, dt_bias, pool, ci, cu, chunk=C, y=y, workspace=ws)
        else:
            gdn.gdn_prefill_gates(a, b, A_log, dt_bias, g, beta)
            gdn.gdn_chunk_prefill(q, k, v, g, beta, pool, ci, cu, chunk=C, y=y, workspace=ws)

    sec = _timed(step, steps, warmup)
    C = min(C, 32) if Dk == 256 else C  # the chunk Dk = 256 runs
    flops = prefill_flops_per_token(Hv, Dk, Dv, C) * T
    return dict(sec=sec, tokens=T, flops=flops, lengths=[int(x) for x in lengths],
                issued=prefill_issued_flops(lengths, Hk, Hv, Dk, Dv, C) if C == 64 else None,
                min_bytes=prefill_min_bytes(T, len(lengths), Hk, Hv, Dk, Dv),
                shape=dict(Hk=Hk, Hv=Hv, Dk=Dk, Dv=Dv, chunk=C, pool=P))


def comba_prefill_min_bytes(T, n_seq, H, K, V, act_bytes=2):
    """Bytes the Comba forward must move: q, k, p, v, o and beta in the
    activation dtype and g (fp32) per token, and each sequence's state slot
    read and written once."""
    per_token = act_bytes * (3 * H * K + 2 * H * V + H) + 4 * H
    return T * per_token + n_seq * 2 * H * K * V * 4


def bench_comba_prefill(steps, warmup, device):
    """comba_chunk_prefill at the varlen token mix with H=32, K=V=128."""
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    from gated_deltanet_linear_gdn_amd import synth
    c = synth.COMBA_PREFILL_VARLEN
    H, K, V, P, C = c["H"], c["K"], c["V"], c["pool"], c["chunk"]
    rng = np.random.default_rng(0)
    lengths = synth.seq_lengths(rng, c["n_seq"], c["len_lo"], c["len_hi"])
    inp = synth.comba_prefill_inputs(rng, lengths, H, K, V, P)
    T = int(inp["cu_seqlens"][-1])
    bf = torch.bfloat16
    d = {n: _dev(inp[n], torch.float32 if n == "g" else bf, device) for n in ("q", "k", "v", "p", "beta", "g")}
    ci = _dev(inp["cache_indices"], torch.int64, device)
    cu = _dev(inp["cu_seqlens"], torch.int64, device)
    pool = torch.zeros((P, H, K, V), dtype=torch.float32, device=device)
    for _ in range(synth.WARMUP_STEPS):  # slots warmed by 16 Comba steps
        t = synth.comba_token(rng, P, H, K, V)
        td = {n: _dev(x, torch.float32 if n == "g" else bf, device) for n, x in t.items()}
        gdn.comba_decode_step(pool, pool, td["q"], td["k"], td["v"], td["p"], td["beta"], td["g"])
    o = torch.empty((T, H, V), dtype=bf, device=device)
    ws = torch.empty(gdn.comba_chunk_prefill_workspace(T, len(lengths), H, K, V, C), dtype=torch.uint8,
                     device=device)

    def step(i):
        gdn.comba_chunk_prefill(d["q"], d["k"], d["v"], d["p"], d["beta"], d["g"], pool, ci, cu, chunk=C,
                                o=o, workspace=ws)

    sec = _timed(step, steps, warmup)
    return dict(sec=sec, tokens=T, flops=prefill_flops_per_token(H, K, V, C) * T,
                issued=prefill_issued_flops(lengths, H, H, K, V, C),
                min_bytes=comba_prefill_min_bytes(T, len(lengths), H, K, V))


def bench_layer(steps, warmup, device):
    """The layer steps around the recurrence at the varlen prefill workload
    (and the decode batch for the conv): conv + SiLU prologue, the gated RMS
    norm epilogue on its own, and the prefill with the norm fused into its
    output against prefill followed by the norm kernel."""
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    from gated_deltanet_linear_gdn_amd import synth
    c = synth.PREFILL_VARLEN
    Hk, Hv, Dk, Dv, P, C = c["Hk"], c["Hv"], c["Dk"], c["Dv"], c["pool"], c["chunk"]
    rng = np.random.default_rng(0)
    lengths = synth.seq_lengths(rng, c["n_seq"], c["len_lo"], c["len_hi"])
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    T = int(inp["cu_seqlens"][-1])
    lay = synth.layer_inputs(rng, T, Hk, Hv, Dk, Dv, P)
    bf = torch.bfloat16
    ci = _dev(inp["cache_indices"], torch.int64, device)
    cu = _dev(inp["cu_seqlens"], torch.int64, device)
    qkv = _dev(lay["qkv"], bf, device)
    w = _dev(lay["conv_w"], torch.float32, device)
    hist = _dev(lay["conv_state"], torch.float32, device)
    z = _dev(lay["z"], bf, device)
    gam = _dev(lay["gamma"], torch.float32, device)
    q = torch.empty((T, Hk, Dk), dtype=bf, device=device)
    k = torch.empty_like(q)
    v = torch.empty((T, Hv, Dv), dtype=bf, device=device)
    a, b = _dev(inp["a"], bf, device), _dev(inp["b"], bf, device)
    g, beta = gdn.gdn_prefill_gates(a, b, _dev(inp["A_log"], torch.float32, device),
                                    _dev(inp["dt_bias"], torch.float32, device))
    pool = torch.zeros((P, Hv, Dv, Dk), dtype=torch.float32, device=device)
    y = torch.empty((T, Hv, Dv), dtype=bf, device=device)
    ws = torch.empty(gdn.gdn_chunk_prefill_workspace(T, len(lengths), Hk, Hv, Dk, Dv, C),
                     dtype=torch.uint8, device=device)
    gdn.gdn_conv_silu(qkv, w, hist, ci, cu, Hk, Hv, Dk, Dv, q, k, v)  # real q/k/v for the prefill
    Cch = 2 * Hk * Dk + Hv * Dv
    conv_sec = _timed(lambda i: gdn.gdn_conv_silu(qkv, w, hist, ci, cu, Hk, Hv, Dk, Dv, q, k, v),
                      steps, warmup)
    norm_sec = _timed(lambda i: gdn.gdn_gated_rmsnorm(y, z, gam, y=y), steps, warmup)
    plain_sec = _timed(lambda i: gdn.gdn_chunk_prefill(q, k, v, g, beta, pool, ci, cu, chunk=C, y=y,
                                                       workspace=ws), steps, warmup)
    fused_sec = _timed(lambda i: gdn.gdn_chunk_prefill(q, k, v, g, beta, pool, ci, cu, chunk=C, y=y,
                                                       workspace=ws, z=z, gamma=gam), steps, warmup)
    # the whole layer prefill from the raw channels: gdn_conv_prefill (conv
    # inside the WY pass) against the separate calls it replaces
    A_log = _dev(inp["A_log"], torch.float32, device)
    dtb = _dev(inp["dt_bias"], torch.float32, device)
    wsc = torch.empty(gdn.gdn_conv_prefill_workspace(T, len(lengths), Hk, Hv, Dk, Dv, C),
                      dtype=torch.uint8, device=device)

    def conv_prefill(z_=None, g_=None):
        gdn.gdn_conv_prefill(qkv, w, hist, a, b, A_log, dtb, pool, ci, cu, Hk, Hv, Dk, Dv, chunk=C, y=y,
                             workspace=wsc, z=z_, gamma=g_)

    def separate(gated):
        gdn.gdn_conv_silu(qkv, w, hist, ci, cu, Hk, Hv, Dk, Dv, q, k, v)
        if gated:
            gdn.gdn_prefill_gates(a, b, A_log, dtb, g, beta)
            gdn.gdn_chunk_prefill(q, k, v, g, beta, pool, ci, cu, chunk=C, y=y, workspace=ws, z=z, gamma=gam)
        else:
            gdn.gdn_chunk_prefill_raw(q, k, v, a, b, A_log, dtb, pool, ci, cu, chunk=C, y=y, workspace=ws)

    cp_sec = _timed(lambda i: conv_prefill(), steps, warmup)
    cp_gated_sec = _timed(lambda i: conv_prefill(z, gam), steps, warmup)
    sep_sec = _timed(lambda i: separate(False), steps, warmup)
    sep_gated_sec = _timed(lambda i: separate(True), steps, warmup)
    # decode step of the conv: one token for each of 256 sequences
    B = synth.DECODE_B256["B"]
    qkv_d = _dev(synth.layer_inputs(rng, B, Hk, Hv, Dk, Dv, 1)["qkv"], bf, device)
    hist_d = torch.zeros((B, Cch, 3), dtype=torch.float32, device=device)
    ci_d = torch.arange(B, dtype=torch.int64, device=device)
    cu_d = torch.arange(B + 1, dtype=torch.int64, device=device)
    qd = torch.empty((B, Hk, Dk), dtype=bf, device=device)
    kd = torch.empty_like(qd)
    vd = torch.empty((B, Hv, Dv), dtype=bf, device=device)
    convd_sec = _timed(lambda i: gdn.gdn_conv_silu(qkv_d, w, hist_d, ci_d, cu_d, Hk, Hv, Dk, Dv, qd, kd, vd),
                       steps, warmup)
    conv_bytes = 2 * T * Cch * 2 + len(lengths) * Cch * 3 * 4 * 2 + Cch * 16
    convd_bytes = 2 * B * Cch * 2 + B * Cch * 3 * 4 * 2 + Cch * 16
    norm_bytes = 3 * T * Hv * Dv * 2 + Dv * 4
    return dict(T=T, conv_sec=conv_sec, conv_bytes=conv_bytes, convd_sec=convd_sec,
                convd_bytes=convd_bytes, norm_sec=norm_sec, norm_bytes=norm_bytes,
                plain_sec=plain_sec, fused_sec=fused_sec, cp_sec=cp_sec, cp_gated_sec=cp_gated_sec,
                sep_sec=sep_sec, sep_gated_sec=sep_gated_sec)


def bench_conv_decode(steps, warmup, device):
    """gdn_conv_decode_step at the B=256 decode batch (conv + SiLU of the
    10,240 raw channels with the history in place, q/k norm, gates and the
    decode step: a q/k prologue kernel and the decode kernel with the value
    channels' conv; states ping-pong between two buffers), and the same
    token through separate kernels: gdn_conv_silu (one token per sequence),
    gdn_prefill_gates and gdn_decode_step (which has no q/k norm, so the
    separate chain does slightly less work)."""
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    from gated_deltanet_linear_gdn_amd import synth
    c = synth.DECODE_B256
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    rng = np.random.default_rng(0)
    bf, f32 = torch.bfloat16, torch.float32
    toks = []
    for _ in range(4):
        d = synth.layer_decode_inputs(rng, B, Hk, Hv, Dk, Dv)
        toks.append({n: _dev(x, f32 if n in ("conv_w", "conv_state", "A_log", "dt_bias") else bf, device)
                     for n, x in d.items()})
    w, A_log, dtb = toks[0]["conv_w"], toks[0]["A_log"], toks[0]["dt_bias"]
    S = [torch.zeros((B, Hv, Dv, Dk), dtype=f32, device=device), torch.empty((B, Hv, Dv, Dk), dtype=f32, device=device)]
    H = toks[0]["conv_state"].clone()
    y = torch.empty((B, Hv, Dv), dtype=bf, device=device)
    ws = torch.empty(gdn.gdn_conv_decode_workspace(B, Hk, Hv, Dk, Dv), dtype=torch.uint8, device=device)

    def fused(i):
        t = toks[i % 4]
        gdn.gdn_conv_decode_step(S[i % 2], S[(i + 1) % 2], t["qkv"], w, H, t["a"], t["b"], A_log, dtb, Hk, y=y,
                                 workspace=ws)

    for i in range(synth.WARMUP_STEPS):
        fused(i)
    fused_sec = _timed(fused, steps, warmup)
    ci = torch.arange(B, dtype=torch.int64, device=device)
    cu = torch.arange(B + 1, dtype=torch.int64, device=device)
    q = torch.empty((B, Hk, Dk), dtype=bf, device=device)
    k = torch.empty_like(q)
    v = torch.empty((B, Hv, Dv), dtype=bf, device=device)
    g = torch.empty((B, Hv), dtype=f32, device=device)
    beta = torch.empty((B, Hv), dtype=f32, device=device)
    beta_act = torch.full((B, Hv), 0.5, dtype=bf, device=device)

    def separate(i):
        t = toks[i % 4]
        gdn.gdn_conv_silu(t["qkv"], w, H, ci, cu, Hk, Hv, Dk, Dv, q, k, v)
        gdn.gdn_prefill_gates(t["a"], t["b"], A_log, dtb, g, beta)
        gdn.gdn_decode_step(S[i % 2], S[(i + 1) % 2], q, k, v, g, beta_act, y)

    sep_sec = _timed(separate, steps, warmup)
    C = 2 * Hk * Dk + Hv * Dv
    state_bytes = 2 * B * Hv * Dv * Dk * 4
    hist_bytes = 2 * B * C * 3 * 4
    return dict(fused_sec=fused_sec, sep_sec=sep_sec, state_bytes=state_bytes,
                bytes=state_bytes + hist_bytes + B * C * 2 + C * 16 + B * Hv * (2 * 2 + Dv * 2))


def bench_comba_hbm(steps, warmup, device, B=896, H=16, K=128, V=128):
    """Comba at one of the KBench measure shapes (0.47-0.94 GB of state per
    copy, beyond the 256 MB MALL)."""
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    from gated_deltanet_linear_gdn_amd import synth
    rng = np.random.default_rng(1)
    toks = []
    for _ in range(4):
        t = synth.comba_token(rng, B, H, K, V)
        toks.append({n: _dev(a, torch.float32 if n == "g" else torch.bfloat16, device)
                     for n, a in t.items()})
    bufs = [torch.zeros((B, H, K, V), dtype=torch.float32, device=device),
            torch.empty((B, H, K, V), dtype=torch.float32, device=device)]
    o = torch.empty((B, H, V), dtype=torch.bfloat16, device=device)

    def step(i):
        t = toks[i % 4]
        gdn.comba_decode_step(bufs[i % 2], bufs[(i + 1) % 2], t["q"], t["k"], t["v"], t["p"],
                              t["beta"], t["g"], o)

    sec = _timed(step, steps, warmup)
    canonical = 2 * B * H * K * V * 4 + B * H * (6 * K + 4 * V + 6)
    return canonical / sec / 1e9, sec


def bench_copy(device, nbytes=2 << 30, reps=20):
    """A 2 GiB device-to-device copy, timed two ways: torch's own copy, and
    the library's one-load, one-store stream copy (gdn_stream_copy, the
    decode step's access pattern).  Returns GB/s over read + write bytes for
    each."""
    import torch
    import gated_deltanet_linear_gdn_amd as gdn
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device=device)
    b = torch.empty_like(a)
    torch_sec = _timed(lambda i: b.copy_(a), reps, 3)
    own_sec = _timed(lambda i: gdn.gdn_stream_copy(a, b), reps, 3)
    assert torch.equal(a, b)
    return 2 * nbytes / torch_sec / 1e9, 2 * nbytes / own_sec / 1e9


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def _run_units(fn, units, threads):
    """fn(unit) for every unit, the units split statically over `threads`
    threads (ctypes releases the GIL inside the oracle).  Returns seconds."""
    import concurrent.futures as cf
    parts = [units[i::threads] for i in range(threads)]
    parts = [p for p in parts if p]
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        list(ex.map(lambda ps: [fn(u) for u in ps], parts))
    return time.perf_counter() - t0


def cpu_baseline(budget_s=8.0):
    """The fp64 oracle (plain C, one token at a time) on this host's cores,
    beside the GPU figures of the same run: the B=256 decode step (the
    headline, GB/s over the same state bytes), the Comba step at B=128
    H=32 K=V=128 (GB/s over the KBench byte count) and the varlen prefill
    (tokens/s over the same 8 sequences x 48 heads), the conv prologue over
    that batch's 10,240 channels and the Comba prefill over the same lengths
    (H=32).  Independent (sequence, head) units (channel blocks for the conv)
    are split statically over N threads; each unit runs sequentially.
    N-thread and 1-thread times are both reported."""
    import oracle
    from gated_deltanet_linear_gdn_amd import synth
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(cores, 64))
    legs = {}

    # decode: whole B=256 steps, batch entries split over the threads
    c = synth.DECODE_B256
    B, Hk, Hv, Dk, Dv = c["B"], c["Hk"], c["Hv"], c["Dk"], c["Dv"]
    rng = np.random.default_rng(1)
    S = np.zeros((B, Hv, Dv, Dk), dtype=np.float64)
    tok = synth.decode_token(rng, B, Hk, Hv, Dk, Dv)

    def dec(b):
        sl = slice(b, b + 1)
        oracle.gdn_step(S[sl], tok["q"][sl], tok["k"][sl], tok["v"][sl], tok["g"][sl], tok["beta"][sl],
                        inplace=True)

    _run_units(dec, list(range(B)), threads)          # first touch of the pages, untimed
    n, el = 0, 0.0
    while el < budget_s and n < 5000:
        el += _run_units(dec, list(range(B)), threads)
        n += 1
    one = _run_units(dec, list(range(B // 8)), 1) * 8  # 1 thread: an eighth of a step, scaled
    state_bytes = 2 * B * Hv * Dv * Dk * 4
    legs["decode"] = dict(workload="gdn_decode_step B=256 Hk=16 Hv=48 Dk=Dv=128", steps=n,
                          s_per_step=round(el / n, 4), s_per_step_1thread=round(one, 4),
                          GBps=round(state_bytes * n / el / 1e9, 3),
                          GBps_1thread=round(state_bytes / one / 1e9, 3))
    del S

    # Comba: whole B=128 H=32 steps
    c = synth.COMBA_B128
    B, H, K, V = c["B"], c["H"], c["K"], c["V"]
    S = np.zeros((B, H, K, V), dtype=np.float64)
    tok = synth.comba_token(rng, B, H, K, V)

    def com(b):
        sl = slice(b, b + 1)
        oracle.comba_step(S[sl], tok["q"][sl], tok["k"][sl], tok["v"][sl], tok["p"][sl], tok["beta"][sl],
                          tok["g"][sl], inplace=True)

    _run_units(com, list(range(B)), threads)
    n, el = 0, 0.0
    while el < budget_s / 4 and n < 5000:
        el += _run_units(com, list(range(B)), threads)
        n += 1
    one = _run_units(com, list(range(B // 8)), 1) * 8
    canonical = 2 * B * H * K * V * 4 + B * H * (6 * K + 4 * V + 6)
    legs["comba"] = dict(workload="comba_decode_step B=128 H=32 K=V=128", steps=n,
                         s_per_step=round(el / n, 4), s_per_step_1thread=round(one, 4),
                         GBps=round(canonical * n / el / 1e9, 3), GBps_1thread=round(canonical / one / 1e9, 3))
    del S

    # varlen prefill: every (sequence, value head) unit of the 8-sequence batch
    c = synth.PREFILL_VARLEN
    Hk, Hv, Dk, Dv, P = c["Hk"], c["Hv"], c["Dk"], c["Dv"], c["pool"]
    rng = np.random.default_rng(0)
    lengths = synth.seq_lengths(rng, c["n_seq"], c["len_lo"], c["len_hi"])
    inp = synth.prefill_inputs(rng, lengths, Hk, Hv, Dk, Dv, pool_size=P)
    g, beta = oracle.gates(inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])
    cu, G = inp["cu_seqlens"], Hv // Hk
    pool = np.zeros((P, Hv, Dv, Dk))

    def pre(u):
        s, hv = u
        idx = slice(int(cu[s]), int(cu[s + 1]))
        hk, h = hv // G, slice(hv, hv + 1)
        slot = int(inp["cache_indices"][s])
        oracle.gdn_prefill(inp["q"][idx, hk:hk + 1], inp["k"][idx, hk:hk + 1], inp["v"][idx, h], g[idx, h],
                           beta[idx, h], pool[slot:slot + 1, h], [0], [0, int(cu[s + 1] - cu[s])])

    units = sorted(((s, hv) for s in range(len(lengths)) for hv in range(Hv)),
                   key=lambda u: -int(lengths[u[0]]))
    T = int(cu[-1])
    el = _run_units(pre, units, threads)
    one_units = [(s, 0) for s in range(len(lengths))]   # 1 thread: head 0 of every sequence, scaled
    one = _run_units(pre, one_units, 1) * Hv
    legs["prefill"] = dict(workload="gdn_chunk_prefill (token by token): 8 sequences of U[512,4096] tokens, "
                                    "Hk=16 Hv=48 Dk=Dv=128", tokens=T, s_per_call=round(el, 3),
                           s_per_call_1thread=round(one, 3), tokens_per_s=round(T / el, 1),
                           tokens_per_s_1thread=round(T / one, 1))

    # the layer prologue over the same batch: conv + SiLU of the 10,240 raw
    # channels, independent channel blocks split over the threads
    lay = synth.layer_inputs(rng, T, Hk, Hv, Dk, Dv, P)
    Cch = lay["qkv"].shape[1]
    blk = Cch // 16

    def conv(j):
        cs = slice(j * blk, (j + 1) * blk)
        oracle.conv_silu(lay["qkv"][:, cs], lay["conv_w"][cs], lay["conv_state"][:, cs], inp["cache_indices"], cu)

    el = _run_units(conv, list(range(16)), threads)
    one = _run_units(conv, [0], 1) * 16
    legs["conv"] = dict(workload="gdn_conv_silu (4-tap conv + SiLU, 10,240 channels, history per slot) over the "
                                 "same 8 sequences", tokens=T, s_per_call=round(el, 3), s_per_call_1thread=round(one, 3),
                        tokens_per_s=round(T / el, 1), tokens_per_s_1thread=round(T / one, 1))

    # Comba prefill: the step over every token of the same 8 sequences, per
    # (sequence, head) unit
    H, K, V = 32, 128, 128
    cin = synth.comba_prefill_inputs(rng, lengths, H, K, V, pool_size=P)
    ccu = cin["cu_seqlens"]
    cpool = np.zeros((P, H, K, V))

    def cpre(u):
        s, h = u
        idx, hs = slice(int(ccu[s]), int(ccu[s + 1])), slice(h, h + 1)
        slot = int(cin["cache_indices"][s])
        oracle.comba_prefill(*(cin[n][idx, hs] for n in ("q", "k", "v", "p", "beta", "g")), cpool[slot:slot + 1, hs],
                             [0], [0, int(ccu[s + 1] - ccu[s])])

    # this oracle steps token by token from Python (one C call per token),
    # so threads serialise on the interpreter: one thread over a sample of
    # two heads of every sequence, scaled to the 32 heads
    one = _run_units(cpre, [(s, h) for s in range(len(lengths)) for h in range(2)], 1) * (H / 2)
    legs["comba_prefill"] = dict(workload="comba_chunk_prefill (token by token): the same 8 sequences, H=32 K=V=128",
                                 tokens=T, sample="heads 0 and 1 of every sequence on 1 thread, scaled by 16",
                                 s_per_call_1thread=round(one, 3), tokens_per_s_1thread=round(T / one, 1))
    d = legs["decode"]
    return dict(value=d["GBps"], unit="GB/s", cores=threads, kind="oracle", cpu=_cpu_model(),
                sample=(f"{d['steps']} fp64 oracle decode steps of the whole B=256 Hk=16 Hv=48 Dk=Dv=128 batch "
                        f"on {threads} threads ({d['s_per_step']} s per step; 1 thread: "
                        f"{d['s_per_step_1thread']} s per step from an eighth of the batch); Comba step, "
                        f"prefill, conv prologue and Comba prefill legs below"),
                legs=legs)


LEGS = ("inplace", "comba", "prefill", "comba_prefill", "dk256", "layer", "conv_decode", "windows", "copy")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma-separated legs to run beside the headline decode "
                    "(for profiling runs): " + ", ".join(LEGS))
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode and prefill kernels shard by "
              "(sequence, head) with no exchange, so the multi-GPU figure is N x the "
              "one-GPU figure at the per-GPU shape; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    device = torch.device("cuda:0")
    dec = bench_decode(args.steps, args.warmup, device)
    only = set(args.only.split(",")) if args.only else None
    want = lambda leg: only is None or leg in only
    if only and not only <= set(LEGS):
        sys.exit(f"--only: unknown legs {sorted(only - set(LEGS))}; known: {', '.join(LEGS)}")
    dec_ip = bench_decode(max(10, args.steps // 2), args.warmup, device, inplace=True) if want("inplace") else None
    dec64 = bench_decode(max(10, args.steps // 2), args.warmup, device, B=64) if want("inplace") else None
    com = bench_comba(args.steps, args.warmup, device) if want("comba") else None
    com_shapes = {}
    if want("comba"):
        from gated_deltanet_linear_gdn_amd import synth as _synth
        for (B_, H_, K_, V_) in _synth.COMBA_MEASURE_SHAPES:
            com_shapes[f"B{B_}_H{H_}_K{K_}_V{V_}"] = bench_comba_hbm(max(10, args.steps // 5), 5, device,
                                                                     B_, H_, K_, V_)
    pre = bench_prefill(max(5, args.steps // 20), 3, device) if want("prefill") else None
    pre_two = bench_prefill(max(5, args.steps // 20), 3, device, raw=False) if want("prefill") else None
    cpre = bench_comba_prefill(max(5, args.steps // 20), 3, device) if want("comba_prefill") else None
    pre256 = bench_prefill(max(5, args.steps // 20), 3, device, Dk=256) if want("dk256") else None
    pre1 = bench_prefill(max(5, args.steps // 20), 3, device, lengths=[4096]) if want("prefill") else None
    dec256 = bench_decode(max(10, args.steps // 5), 5, device, B=128, Dk=256) if want("dk256") else None
    lay = bench_layer(max(5, args.steps // 50), 3, device) if want("layer") else None
    cdec = bench_conv_decode(max(10, args.steps // 5), 5, device) if want("conv_decode") else None
    wins = ({T: bench_window(max(10, args.steps // 5), 5, device, T) for T in (2, 4, 8)}
            if want("windows") else None)
    cwins = ({T: bench_window(max(10, args.steps // 5), 5, device, T, chunked=True) for T in (4, 8, 16, 64)}
             if want("windows") else None)
    vwins = ({(T, ch): bench_window(max(10, args.steps // 5), 5, device, T, chunked=ch, verify=True)
              for T in (4, 8, 16) for ch in (False, True) if ch or T <= 8}
             if want("windows") else None)
    copy_gbps, own_copy_gbps = bench_copy(device) if want("copy") else (None, None)

    gbps = dec["state_bytes"] / dec["sec"] / 1e9
    out = {
        "metric": "decode state GB/s (% of HBM peak); chunked-prefill tokens/s (% MFMA peak)",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["sec"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "gdn_decode_step, large decode batch: B=256 Hk=16 Hv=48 Dk=Dv=128, "
                               "bf16 q/k/v/beta, fp32 g and state (0.8 GB), functional state_in -> state_out",
                   **dec["shape"], "state_bytes_per_step": dec["state_bytes"],
                   "activation_bytes_per_step": dec["act_bytes"]},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": _decode_traffic(),
                     "traffic_source": ("stored figure from two earlier rocprofv3 --pmc runs (FETCH_SIZE x 2 + "
                                        "WRITE_SIZE x 1) of this kernel, reported only while its sources hash "
                                        "to the values recorded with it; not read in this run")},
    }
    if want("inplace"):
        out["decode_inplace_GBps"] = round(dec_ip["state_bytes"] / dec_ip["sec"] / 1e9, 2)
        out["decode_b64"] = {"workload": "gdn_decode_step, decode batch B=64 Hk=16 Hv=48 Dk=Dv=128 bf16, fp32 state "
                                         "(192 MiB per copy, functional ping-pong: 384 MiB, above the 256 MB MALL, "
                                         "which still holds part of it between steps)",
                             "us_per_step": round(dec64["sec"] * 1e6, 2),
                             "GBps": round(dec64["state_bytes"] / dec64["sec"] / 1e9, 2),
                             "frac_of_hbm_peak": round(dec64["state_bytes"] / dec64["sec"] / 1e9 / HBM_PEAK_GBPS, 4)}
    if want("copy"):
        out["torch_copy_GBps"] = round(copy_gbps, 1)
    if want("copy"):
        out["stream_copy"] = {"workload": "gdn_stream_copy of 2 GiB: one 16-byte non-temporal load and store per "
                                         "thread, the decode step's access pattern (GB/s over read + write bytes)",
                             "GBps": round(own_copy_gbps, 1),
                             "frac_of_hbm_peak": round(own_copy_gbps / HBM_PEAK_GBPS, 4),
                             "decode_frac_of_copy": round(gbps / own_copy_gbps, 4)}
    if want("windows"):
        out["decode_window"] = {"workload": "gdn_decode_window at the B=256 decode batch, all T tokens committed",
                               "tokens_per_s_single_step": round(dec["shape"]["B"] / dec["sec"], 1),
                               **{f"T{T}": {"us_per_window": round(w["sec"] * 1e6, 2),
                                            "tokens_per_s": round(w["tokens"] / w["sec"], 1),
                                            "state_GBps": round(w["state_bytes"] / w["sec"] / 1e9, 1)}
                                  for T, w in wins.items()},
                               "chunked": {"workload": "the same committed windows as gdn_chunk_prefill_fixed "
                                                       "(no norm, scale 1, chunk min(T, 64)), in place",
                                           **{f"T{T}": {"us_per_window": round(w["sec"] * 1e6, 2),
                                                        "tokens_per_s": round(w["tokens"] / w["sec"], 1),
                                                        "state_GBps": round(w["state_bytes"] / w["sec"] / 1e9, 1)}
                                              for T, w in cwins.items()}},
                               "verify": {"workload": "verify windows (every y, nothing committed, the state only "
                                                      "read): gdn_decode_window with commit 0, and chunked as "
                                                      "gdn_chunk_prefill_fixed with GDN_KEEP_STATE",
                                          **{f"{'chunked_' if ch else ''}T{T}": {
                                              "us_per_window": round(w["sec"] * 1e6, 2),
                                              "tokens_per_s": round(w["tokens"] / w["sec"], 1),
                                              "state_GBps": round(w["state_bytes"] / w["sec"] / 1e9, 1)}
                                             for (T, ch), w in vwins.items()}}}
    if want("comba"):
        out["comba"] = {"workload": "comba_decode_step B=128 H=32 K=V=128 bf16, fp32 state",
                       "GBps": round(com["bytes"] / com["sec"] / 1e9, 2),
                       "us_per_step": round(com["sec"] * 1e6, 2),
                       "frac_of_hbm_peak": round(com["bytes"] / com["sec"] / 1e9 / HBM_PEAK_GBPS, 4),
                       "measure_shapes": {name: {"GBps": round(gbps, 2), "us_per_step": round(sec * 1e6, 2),
                                                 "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
                                          for name, (gbps, sec) in com_shapes.items()}}
    if want("conv_decode"):
        out["conv_decode"] = {"workload": "gdn_conv_decode_step at B=256 Hk=16 Hv=48 Dk=Dv=128 bf16: conv + SiLU of "
                                         "10,240 raw channels (history in place), q/k norm and gates in a prologue "
                                         "kernel (fp32 results to a workspace), then the decode kernel; states "
                                         "ping-pong",
                             "us_per_step": round(cdec["fused_sec"] * 1e6, 2),
                             "GBps": round(cdec["bytes"] / cdec["fused_sec"] / 1e9, 1),
                             "state_GBps": round(cdec["state_bytes"] / cdec["fused_sec"] / 1e9, 1),
                             "separate_kernels_us_per_step": round(cdec["sep_sec"] * 1e6, 2),
                             "bytes_per_step": cdec["bytes"]}
    if want("prefill"):
        out["prefill"] = {"workload": "gdn_chunk_prefill_raw (gates from raw a, b, A_log, dt_bias formed inside "
                                     "the WY pass), 8 sequences of U[512,4096] tokens, Hk=16 Hv=48 Dk=Dv=128, bf16, "
                                     "chunk 64, pool 16",
                         "two_calls_us_per_call": round(pre_two["sec"] * 1e6, 2),
                         "tokens": pre["tokens"], "lengths": pre["lengths"],
                         "us_per_call": round(pre["sec"] * 1e6, 2),
                         "tokens_per_s": round(pre["tokens"] / pre["sec"], 1),
                         "canonical_TFLOPs": round(pre["flops"] / pre["sec"] / 1e12, 2),
                         "mfma_frac_of_bf16_peak": round(pre["flops"] / pre["sec"] / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "issued_mfma_frac_of_bf16_peak": round(pre["issued"] / pre["sec"] / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "min_bytes": pre["min_bytes"],
                         "hbm_frac_of_peak": round(pre["min_bytes"] / pre["sec"] / 1e9 / HBM_PEAK_GBPS, 4)}
    if want("prefill"):
        out["prefill_single"] = {"workload": "gdn_chunk_prefill_raw of one 4,096-token sequence "
                                            "(the workload's longest length), Hk=16 Hv=48 Dk=Dv=128, bf16, chunk 64",
                                "us_per_call": round(pre1["sec"] * 1e6, 2),
                                "tokens_per_s": round(pre1["tokens"] / pre1["sec"], 1)}
    if want("comba_prefill"):
        out["comba_prefill"] = {"workload": "comba_chunk_prefill, the same 8 sequences, H=32 K=V=128, bf16, "
                                           "chunk 64, pool 16",
                               "tokens": cpre["tokens"],
                               "us_per_call": round(cpre["sec"] * 1e6, 2),
                               "tokens_per_s": round(cpre["tokens"] / cpre["sec"], 1),
                               "canonical_TFLOPs": round(cpre["flops"] / cpre["sec"] / 1e12, 2),
                               "mfma_frac_of_bf16_peak": round(cpre["flops"] / cpre["sec"] / 1e12 / BF16_PEAK_TFLOPS, 4),
                               "issued_mfma_frac_of_bf16_peak": round(cpre["issued"] / cpre["sec"] / 1e12
                                                                      / BF16_PEAK_TFLOPS, 4),
                               "min_bytes": cpre["min_bytes"],
                               "hbm_frac_of_peak": round(cpre["min_bytes"] / cpre["sec"] / 1e9 / HBM_PEAK_GBPS, 4)}
    if want("dk256"):
        out["dk256"] = {"workload": "key head size 256 (value 128): gdn_chunk_prefill_raw at the varlen token mix "
                                   "(Hk=16 Hv=48, 32-token chunks) and gdn_decode_step at B=128 (the same "
                                   "1.6 GB of state per step as the headline)",
                       "prefill_us_per_call": round(pre256["sec"] * 1e6, 2),
                       "prefill_tokens_per_s": round(pre256["tokens"] / pre256["sec"], 1),
                       "prefill_canonical_TFLOPs": round(pre256["flops"] / pre256["sec"] / 1e12, 2),
                       "decode_GBps": round(dec256["state_bytes"] / dec256["sec"] / 1e9, 2),
                       "decode_frac_of_hbm_peak": round(dec256["state_bytes"] / dec256["sec"] / 1e9
                                                        / HBM_PEAK_GBPS, 4)}
    if want("layer"):
        out["layer"] = {"workload": "prologue gdn_conv_silu (4-tap conv + SiLU, 10,240 channels, history per "
                                   "slot) and epilogue gdn_gated_rmsnorm around the varlen prefill; conv "
                                   "also as a decode step of 256 sequences",
                       "conv_us": round(lay["conv_sec"] * 1e6, 2),
                       "conv_GBps": round(lay["conv_bytes"] / lay["conv_sec"] / 1e9, 1),
                       "conv_decode_B256_us": round(lay["convd_sec"] * 1e6, 2),
                       "conv_decode_B256_GBps": round(lay["convd_bytes"] / lay["convd_sec"] / 1e9, 1),
                       "norm_us": round(lay["norm_sec"] * 1e6, 2),
                       "norm_GBps": round(lay["norm_bytes"] / lay["norm_sec"] / 1e9, 1),
                       "prefill_us": round(lay["plain_sec"] * 1e6, 2),
                       "prefill_gated_fused_us": round(lay["fused_sec"] * 1e6, 2),
                       "prefill_then_norm_us": round((lay["plain_sec"] + lay["norm_sec"]) * 1e6, 2),
                       "conv_prefill": {
                           "workload": "gdn_conv_prefill: conv + SiLU inside the WY pass, gates from raw a, b, "
                                       "the chunked recurrence (and the gated norm) in one call, against "
                                       "gdn_conv_silu + gdn_chunk_prefill_raw (and gdn_conv_silu + "
                                       "gdn_prefill_gates + the gated gdn_chunk_prefill) timed as one step",
                           "us_per_call": round(lay["cp_sec"] * 1e6, 2),
                           "separate_us_per_call": round(lay["sep_sec"] * 1e6, 2),
                           "gated_us_per_call": round(lay["cp_gated_sec"] * 1e6, 2),
                           "separate_gated_us_per_call": round(lay["sep_gated_sec"] * 1e6, 2),
                           "tokens_per_s": round(lay["T"] / lay["cp_sec"], 1),
                           "gated_tokens_per_s": round(lay["T"] / lay["cp_gated_sec"], 1)}}
    if not args.no_cpu_baseline and only is None:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
