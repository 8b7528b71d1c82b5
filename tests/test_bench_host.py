"""Host-side checks of bench.py: the work and byte accounting it reports
beside the timings, and the one-GPU guard.  No GPU needed."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_canonical_flops_per_token():
    # 6 Dk Dv + C (6 Dk + 4 Dv) per value head: 180,224 at D = 128, C = 64
    assert bench.prefill_flops_per_token(1, 128, 128, 64) == 180_224
    assert bench.prefill_flops_per_token(48, 128, 128, 64) == 48 * 180_224


def test_prefill_min_bytes_per_token():
    # q, k (16 heads x 128) and v, y (48 heads x 128) in bf16, plus a and b
    # (48 heads, bf16): 32,960 bytes per token; plus 3 MiB of state per
    # sequence in each direction
    one_token = bench.prefill_min_bytes(1, 0, 16, 48, 128, 128)
    assert one_token == 32_960
    assert bench.prefill_min_bytes(0, 1, 16, 48, 128, 128) == 2 * 3 * 2**20


def test_prefill_issued_flops_single_chunk():
    # one full chunk, one key head with one value head, D = 128, C = 64
    f = bench.prefill_issued_flops([64], 1, 1, 128, 128, 64)
    mfma32 = 16 * 16 * 32 * 2   # one 16x16x32 product
    mfma16 = 16 * 16 * 16 * 2   # one 16x16x16 product
    # chunk loop: 8 waves x (64 phase A: X and Y with S as hi + lo; 18 phase
    # B + 6 P Delta + 32 update)
    loop = 8 * 120 * mfma32
    # WY: 10 lower 16x16 blocks x 4 k-steps x (K K^T, Q K^T); 16 steps of the
    # blocked inverse x 3 hi/lo products
    wy = 10 * 4 * 2 * mfma32 + 16 * 3 * mfma16
    assert f == loop + wy
    # a ragged sequence counts its partial chunk as a whole one
    assert bench.prefill_issued_flops([65], 1, 1, 128, 128, 64) == 2 * f


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_comba_prefill_min_bytes_per_token():
    # q, k, p (32 heads x 128), v, o (32 x 128) and beta (32) in bf16, g (32)
    # in fp32: 2 * (3*4096 + 2*4096 + 32) + 128 = 41,152 bytes per token
    assert bench.comba_prefill_min_bytes(1, 0, 32, 128, 128) == 41_152
    assert bench.comba_prefill_min_bytes(0, 1, 32, 128, 128) == 2 * 32 * 128 * 128 * 4
