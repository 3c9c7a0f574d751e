"""GPU parity of every matrix-core tile shape, forced through w4a16_set_tile.

The default planner picks one tile per problem; these tests run the other
shapes (split-K over 1-8 waves, waves owning 1-4 tiles) on shapes that reach
their edge cases: several activation slices per wave, ragged last K range,
8-scale vector loads and the one-scale path, gathered rows with invalid ids,
and the argmax partials of each workgroup shape.  Expected values come only
from the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, dev, forced_tile, host, say, sample_rows, weight_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TILES = ["split,1,1", "split,1,8", "split,2,3", "split,4,2", "shared,1,1", "shared,2,3", "shared,4,4", "shared,1,16",
         "run,3,4", "run,2,16"]

# (N, K, T): single group; odd rows; several slices at T = 8 (G = 136); a
# ragged tile tail; G = 18 (one scale per load); a tall K = 5120 case.
SHAPES = [(1, 128, 1), (37, 1152, 3), (300, 17408, 8), (1003, 640, 5), (2000, 2304, 8), (4099, 5120, 4)]


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    w4a16.set_variant("mfma")
    yield w4a16
    w4a16.set_variant("auto")


@pytest.mark.parametrize("tile", TILES)
def test_tile_shapes_match_oracle(w4, tile):
    with forced_tile(w4, tile):
        for N, K, T in SHAPES:
            say(f"tile {tile} N={N} K={K} T={T}")
            tid = 3000 + N + K + T
            p, s, pd, sd = weight_dev(tid, N, K)
            x = synth.activations(tid, T, K)
            y_ref, a_ref = oracle.matmul(p, s, x)
            assert_parity(host(w4.matmul(pd, sd, dev(x))), y_ref, a_ref, f"{tile} N={N} K={K} T={T}")


@pytest.mark.parametrize("tile", TILES)
def test_tile_misaligned_scales(w4, tile):
    """Scale rows 2 bytes past 16-byte alignment take the one-scale-per-load path."""
    with forced_tile(w4, tile):
        N, K, T = 520, 2048, 3
        p, s = synth.weight(3100, N, K)
        x = synth.activations(3100, T, K)
        buf = torch.empty(s.size + 8, dtype=torch.int16, device="cuda")
        sd = buf[1:1 + s.size].view(N, K // 128)
        sd.copy_(dev(s))
        assert sd.data_ptr() % 16 == 2
        y_ref, a_ref = oracle.matmul(p, s, x)
        assert_parity(host(w4.matmul(dev(p), sd, dev(x))), y_ref, a_ref, f"{tile} misaligned scales")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("T", [2, 8])
def test_tile_gather_argmax(w4, tile, T):
    with forced_tile(w4, tile):
        N, K = 3000, 1280
        p, s, pd, sd = weight_dev(3200 + T, N, K)
        x = synth.activations(3200 + T, T, K)
        rng = np.random.default_rng(T)
        ids = rng.integers(0, N, 1500).astype(np.int32)
        ids[[3, 700, 1499]] = [-1, N, 2**31 - 1]
        y, am, av = w4.head_gather(pd, sd, dev(x), row_ids=dev(ids), scores=True, argmax=True)
        y, am, av = host(y), host(am), host(av)
        y_ref, a_ref = oracle.gather(ids, p, s, x)
        assert_parity(y, y_ref, a_ref, f"{tile} gather T={T}")
        # the GPU's own scores decide the argmax; the oracle's must agree up to a near-tie
        id_ref, val_ref, _ = oracle.argmax(y_ref, ids)
        for t in range(T):
            valid = ~np.isnan(y[t])
            best = np.max(y[t][valid])
            cand = ids[valid][y[t][valid] == best]
            assert am[t] == cand.min(), f"{tile} T={T} t={t}: id {am[t]} vs {cand.min()}"
            assert av[t] == best
            if am[t] != id_ref[t]:
                j = np.flatnonzero(ids == am[t])[0]
                k = np.flatnonzero(ids == id_ref[t])[0]
                gap = abs(y_ref[t, j] - y_ref[t, k])
                assert gap <= 1e-3 * (a_ref[t, j] + a_ref[t, k]), f"{tile} T={T} t={t}: not a near-tie"
