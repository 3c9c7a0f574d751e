"""GPU parity at seeded random shapes: every planner branch (split, shared and
run tilings, the dot variant, both layouts, the grouped launch with mixed
problems) on sizes that no hand-picked case names, against the oracle.

Shapes are drawn from a fixed seed: N from a few rows to several thousand
(ragged against the 16-row tiles), K from one group to 136 groups (ragged
against the 8-group load ring), T from 1 to 16.  Rows are compared in full
up to 2,048 rows, else on a sample that includes the tile edges.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, dev, host, sample_rows, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CASES = 16


def draw_shapes(seed: int, count: int):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        band = rng.integers(0, 3)
        N = int(rng.integers(1, 64) if band == 0 else rng.integers(64, 1500) if band == 1 else rng.integers(1500, 5000))
        G = int(rng.choice([rng.integers(1, 12), rng.integers(12, 48), 136]))
        out.append((N, 128 * G, int(rng.integers(1, 17))))
    return out


SHAPES = draw_shapes(20261202, N_CASES)


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    yield w4a16
    w4a16.set_variant("auto")


def reference(p, s, x):
    N = p.shape[0]
    rows = np.arange(N, dtype=np.int32) if N <= 2048 else sample_rows(N, 256, seed=N)
    y_ref, a_ref = oracle.gather(rows, p, s, x)
    return rows, y_ref, a_ref


@pytest.mark.parametrize("case", range(N_CASES))
@pytest.mark.parametrize("path", ["mfma", "dot", "tiled"])
def test_random_shape_single_launch(w4, case, path):
    N, K, T = SHAPES[case]
    say(f"random single {path} N={N} K={K} T={T}")
    p, s = synth.weight(7000 + case, N, K)
    x = synth.activations(7000 + case, T, K)
    pd, sd, xd = dev(p), dev(s), dev(x)
    if path == "tiled":
        y = w4.matmul_tiled(w4.repack_tiled(pd, sd), xd)
    else:
        w4.set_variant(path)
        y = w4.matmul(pd, sd, xd)
        w4.set_variant("auto")
    rows, y_ref, a_ref = reference(p, s, x)
    assert_parity(host(y)[:, rows], y_ref, a_ref, f"{path} N={N} K={K} T={T}")


@pytest.mark.parametrize("layouts", ["tiled", "row-major", "mixed"])
@pytest.mark.parametrize("T", [2, 6, 11])
def test_random_shapes_grouped(w4, layouts, T):
    """Ten random problems in one grouped launch (all tiled: run workgroups;
    some row-major: shared workgroups), run twice with the same result."""
    rng = np.random.default_rng(100 * T + len(layouts))
    probs, host_side = [], []
    for i in range(10):
        N, K, _ = SHAPES[int(rng.integers(0, N_CASES))]
        tid = 7100 + 10 * T + i
        p, s = synth.weight(tid, N, K)
        x = synth.activations(tid, T, K)
        pd, sd = dev(p), dev(s)
        tiled = layouts == "tiled" or (layouts == "mixed" and i % 2 == 0)
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        probs.append((w4.repack_tiled(pd, sd), None, dev(x), y) if tiled else (pd, sd, dev(x), y))
        host_side.append((p, s, x))
    say(f"random grouped {layouts} T={T}: " + ", ".join(f"{p.shape[0]}x{p.shape[1] * 2}" for p, _, _ in host_side))
    b = w4.Batch(probs, T)
    b.run()
    first = []
    for (*_, y), (p, s, x) in zip(probs, host_side):
        rows, y_ref, a_ref = reference(p, s, x)
        yh = host(y)
        assert_parity(yh[:, rows], y_ref, a_ref, f"grouped {layouts} T={T} N={p.shape[0]} K={p.shape[1] * 2}")
        first.append(yh.copy())
    b.run()
    for f, (*_, y) in zip(first, probs):
        assert np.array_equal(f, host(y)), "second run differs"
