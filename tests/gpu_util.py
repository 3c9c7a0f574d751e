"""Shared helpers of the GPU parity tests (host-side comparison only)."""
import contextlib
import sys

import numpy as np
import torch

import oracle
import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def forced_tile(w4, spec, batch: bool = False):
    """Runs the body with the tiling of single launches (batch=True: grouped
    launches) forced to `spec` through the library's run-time override, then
    gives the choice back to the planner.  (W4A16_TILE / W4A16_BATCH_TILE are
    read once per process, at the first plan: setting them inside a test does
    not reach the library.)"""
    w4.set_tile(spec, batch=batch)
    try:
        yield
    finally:
        w4.set_tile(None, batch=batch)


def batch_variant(b) -> int:
    """The kernel shape a grouped launch's table records (2 split, 3 shared,
    4 runs of tiles): the fifth 32-bit word of its header."""
    return int(b.host[16:20].view(torch.int32)[0])


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


# Near-tie exemptions taken by check_argmax in this process (reported by each
# call and in the session summary of conftest.py).
NEAR_TIES = []


def check_argmax(ids_gpu, y_gpu_full, y_ref, ids_map, what) -> int:
    """GPU argmax vs (a) the host argmax over the GPU's own scores, bit-exact,
    and (b) the oracle's argmax, exact unless the oracle's gap between its
    best id and the best other id is below the GPU's measured error on those
    two rows.  Returns the number of rows that took that exemption."""
    ids_gpu = np.asarray(ids_gpu)
    y_gpu_full = np.asarray(y_gpu_full, dtype=np.float64)
    T = y_ref.shape[0]
    own_id, _, _ = oracle.argmax(y_gpu_full, ids_map)
    assert np.array_equal(ids_gpu, own_id), f"{what}: GPU argmax != host argmax of GPU scores"
    ref_id, _, gap = oracle.argmax(y_ref, ids_map)
    taken = 0
    for t in range(T):
        if ids_gpu[t] == ref_id[t]:
            continue
        assert ids_gpu[t] >= 0 and ref_id[t] >= 0, f"{what}: t={t}: {ids_gpu[t]} vs oracle {ref_id[t]}"
        pos = {int(v): i for i, v in enumerate(ids_map if ids_map is not None else range(y_ref.shape[1]))}
        i_g, i_r = pos[int(ids_gpu[t])], pos[int(ref_id[t])]
        err = abs(y_gpu_full[t, i_g] - y_ref[t, i_g]) + abs(y_gpu_full[t, i_r] - y_ref[t, i_r])
        assert gap[t] < err, f"{what}: argmax {ids_gpu[t]} != oracle {ref_id[t]} (gap {gap[t]}, err {err})"
        taken += 1
        NEAR_TIES.append((what, t, float(gap[t]), float(err)))
    say(f"  {what}: argmax checked on {T} rows, {taken} near-tie exemption(s)")
    return taken
