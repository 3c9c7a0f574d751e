"""Shared helpers of the GPU parity tests (host-side comparison only)."""
import sys

import numpy as np
import torch

import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    """Host array -> contiguous CUDA tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def tolerance(a_ref: np.ndarray) -> np.ndarray:
    """Per-element bound |y_gpu - y_ref| <= 1e-3 * sum_k |w*x| + 1e-6."""
    return 1e-3 * a_ref + 1e-6


def assert_parity(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, what: str) -> float:
    """Element-by-element check; NaN expected exactly where the oracle has NaN."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y_gpu), nan_ref), f"{what}: NaN pattern differs"
    ok = ~nan_ref
    err = np.abs(y_gpu[ok] - y_ref[ok])
    tol = tolerance(a_ref[ok])
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, first at {idx.ravel().tolist()}: "
                             f"gpu {y_gpu[ok][bad][:3]} ref {y_ref[ok][bad][:3]} tol {tol[bad][:3]}")
    return float((err / tol).max()) if err.size else 0.0


def weight_dev(tid, n, k):
    p, s = synth.weight(tid, n, k)
    return p, s, dev(p), dev(s)


def sample_rows(n: int, count: int, seed: int) -> np.ndarray:
    """Sorted sample of row indices including both ends and tile edges."""
    rng = np.random.default_rng(seed)
    base = rng.choice(n, size=min(count, n), replace=False)
    edges = np.array([0, 1, 15, 16, 17, 63, 64, n // 2, n - 17, n - 16, n - 2, n - 1])
    edges = edges[(edges >= 0) & (edges < n)]
    return np.unique(np.concatenate([base, edges])).astype(np.int32)
