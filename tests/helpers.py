"""Test helpers: error measures, host<->device moves, threaded oracle calls."""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle


def maxrel(x, ref) -> float:
    """max |x - ref| / max |ref| over the whole tensor."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(x - ref))) / (den if den > 0 else 1.0) if ref.size else 0.0


def relF(x, ref) -> float:
    """||x - ref||_F / ||ref||_F (the KBench spec's correctness measure)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    return float(np.linalg.norm((x - ref).ravel())) / (den if den > 0 else 1.0)


def rowrel(x, ref, floor=1e-3) -> float:
    """Largest error of one output row (the last axis): over every row,
    max |x - ref| in the row / max |ref| in the row.  Rows whose largest
    element is below `floor` times the tensor's largest are measured against
    that floor, so a row that is nearly zero in the reference does not turn
    fp32 rounding into a large ratio."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return 0.0
    n = ref.shape[-1]
    err = np.max(np.abs(x - ref).reshape(-1, n), axis=1)
    scale = np.max(np.abs(ref).reshape(-1, n), axis=1)
    top = float(np.max(scale))
    den = np.maximum(scale, floor * top if top > 0 else 1.0)
    return float(np.max(err / den))


def check_bf16_out(x, ref, what="output"):
    """A bf16 output against the fp64 oracle, element by element: relative
    Frobenius error <= 2e-2, max |error| <= 1e-2 of the largest reference
    value, and in every row max |error| <= 2e-2 of that row's largest value
    (the 2e-2 relative bound of a bf16 output, applied row by row; rounding
    to bf16 alone gives at most 2^-9 ~ 2e-3 of an element).  With
    GDN_TEST_ERRLOG set, the three figures are appended to that file."""
    e = (relF(x, ref), maxrel(x, ref), rowrel(x, ref))
    log = os.environ.get("GDN_TEST_ERRLOG")
    if log:
        with open(log, "a") as f:
            f.write(f"{os.environ.get('PYTEST_CURRENT_TEST', '?').split(' ')[0]} {what}: "
                    f"relF {e[0]:.3e} maxrel {e[1]:.3e} rowrel {e[2]:.3e}\n")
    assert e[0] <= 2e-2 and e[1] <= 1e-2 and e[2] <= 2e-2, f"{what}: relF {e[0]:.3g}, maxrel {e[1]:.3g}, rowrel {e[2]:.3g}"
    return e


def to_dev(x, dtype, device):
    """numpy float32/int64 -> torch tensor on device.  float32 values that are
    bf16-representable convert exactly (round-to-nearest-even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=device, dtype=dtype).contiguous()


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(dtype=torch.float64 if t.is_floating_point() else t.dtype).cpu().numpy()


def n_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _split_batch(B, threads):
    parts = np.array_split(np.arange(B), min(threads, max(B, 1)))
    return [slice(int(p[0]), int(p[-1]) + 1) for p in parts if p.size]


def oracle_decode_batched(S, tok, threads=None):
    """oracle.gdn_step, updating the float64 state S IN PLACE, split over the
    batch across threads (ctypes releases the GIL; batch entries are
    independent).  Returns (S, y)."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    y = np.empty(tok["v"].shape, dtype=np.float64)

    def run(sl):
        _, y[sl] = oracle.gdn_step(S[sl], tok["q"][sl], tok["k"][sl], tok["v"][sl],
                                   tok["g"][sl], tok["beta"][sl], inplace=True)

    with cf.ThreadPoolExecutor(max_workers=threads or n_threads()) as ex:
        list(ex.map(run, _split_batch(S.shape[0], threads or n_threads())))
    return S, y


def oracle_comba_batched(S, tok, scale=None, threads=None):
    """oracle.comba_step, in place on the float64 state S, threaded over B."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    o = np.empty(tok["v"].shape, dtype=np.float64)

    def run(sl):
        _, o[sl] = oracle.comba_step(S[sl], tok["q"][sl], tok["k"][sl], tok["v"][sl],
                                     tok["p"][sl], tok["beta"][sl], tok["g"][sl], scale=scale,
                                     inplace=True)

    with cf.ThreadPoolExecutor(max_workers=threads or n_threads()) as ex:
        list(ex.map(run, _split_batch(S.shape[0], threads or n_threads())))
    return S, o
