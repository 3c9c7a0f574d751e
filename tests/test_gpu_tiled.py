"""GPU parity of the tiled weight layout.

The repack is checked byte for byte against the layout written out here
from its definition in include/w4a16.h (numpy, no library code); the
matmul, gathered head and grouped launch on tiled weights are checked
against the oracle on the original row-major weight.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, check_argmax, dev, forced_tile, host, say, sample_rows, weight_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    return w4a16


def layout_by_definition(p: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Tiles of 16 rows; chunks of up to 8 groups; a group = 16 rows x 64 code
    bytes in row order; after a chunk's codes, 16 rows x 8 bf16 scales."""
    N, kh = p.shape
    G = 2 * kh // 128
    C = -(-G // 8)
    tiles = -(-N // 16)
    tile_bytes = G * 1024 + C * 256
    pp = np.zeros((tiles * 16, kh), np.uint8)
    pp[:N] = p
    ss = np.zeros((tiles * 16, C * 8), np.uint16)
    ss[:N, :G] = s
    out = np.zeros(tiles * tile_bytes, np.uint8)
    for i in range(tiles):
        for c in range(C):
            ng = min(8, G - 8 * c)
            cb = i * tile_bytes + c * (8 * 1024 + 256)
            for gi in range(ng):
                g = 8 * c + gi
                out[cb + gi * 1024: cb + (gi + 1) * 1024] = pp[16 * i:16 * i + 16, 64 * g:64 * g + 64].reshape(-1)
            sc = np.ascontiguousarray(ss[16 * i:16 * i + 16, 8 * c:8 * c + 8]).astype("<u2")
            out[cb + ng * 1024: cb + ng * 1024 + 256] = sc.view(np.uint8).reshape(-1)
    return out


@pytest.mark.parametrize("N,K", [(16, 128), (37, 1152), (300, 5120), (33, 2048)])
def test_repack_matches_layout_definition(w4, N, K):
    p, s, pd, sd = weight_dev(4000 + N + K, N, K)
    tw = w4.repack_tiled(pd, sd)
    assert tw.data.numel() == w4.tiled_bytes(N, K)
    got = host(tw.data)
    want = layout_by_definition(p, s)
    assert got.shape == want.shape
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"N={N} K={K}: {bad.size} bytes differ, first at {bad[:5]}"


TILED_SHAPES = [(1, 128, 1), (17, 384, 3), (37, 1152, 8), (1003, 640, 2), (4099, 1280, 4), (257, 5120, 7),
                (31, 17408, 8), (16400, 1024, 1), (17003, 1152, 3), (16413, 2304, 8), (300, 17408, 5)]


@pytest.mark.parametrize("N,K,T", TILED_SHAPES)
def test_matmul_tiled_matches_oracle(w4, N, K, T):
    say(f"tiled N={N} K={K} T={T}")
    tid = 4100 + N + K + T
    p, s, pd, sd = weight_dev(tid, N, K)
    x = synth.activations(tid, T, K)
    tw = w4.repack_tiled(pd, sd)
    y_ref, a_ref = oracle.matmul(p, s, x)
    assert_parity(host(w4.matmul_tiled(tw, dev(x))), y_ref, a_ref, f"tiled N={N} K={K} T={T}")


@pytest.mark.parametrize("tile", ["split,1,8", "split,2,3", "split,2,8", "shared,1,1", "shared,4,8", "shared,2,4", "shared,1,16", "shared,1,12", "run,4,8", "run,2,16"])
def test_matmul_tiled_every_tile_shape(w4, tile):
    with forced_tile(w4, tile):
        for N, K, T in [(37, 1152, 3), (300, 17408, 8), (2000, 2304, 8), (4099, 5120, 4)]:
            tid = 4200 + N + K + T
            p, s, pd, sd = weight_dev(tid, N, K)
            x = synth.activations(tid, T, K)
            y_ref, a_ref = oracle.matmul(p, s, x)
            y = host(w4.matmul_tiled(w4.repack_tiled(pd, sd), dev(x)))
            assert_parity(y, y_ref, a_ref, f"{tile} tiled N={N} K={K} T={T}")


@pytest.mark.parametrize("proj", synth.PROJ_ORDER)
def test_projection_tiled_sampled(w4, proj):
    N, K = synth.PROJECTIONS[proj]
    p, s, pd, sd = weight_dev(synth.tid_layer(5, proj), N, K)
    tw = w4.repack_tiled(pd, sd)
    del pd, sd
    rows = sample_rows(N, 300, seed=N + 1)
    for T in (1, 4, 8):
        say(f"tiled {proj} T={T}")
        x = synth.activations(synth.tid_layer(5, proj) + 100, T, K)
        y = host(w4.matmul_tiled(tw, dev(x)))
        y_ref, a_ref = oracle.gather(rows, p, s, x)
        assert_parity(y[:, rows], y_ref, a_ref, f"tiled {proj} T={T}")


def test_gather_tiled_bad_ids_and_argmax(w4):
    N, K, T = 3000, 1152, 4
    p, s, pd, sd = weight_dev(4300, N, K)
    x = synth.activations(4300, T, K)
    tw = w4.repack_tiled(pd, sd)
    ids = np.random.default_rng(3).integers(0, N, 1200).astype(np.int32)
    ids[[0, 599, 1199]] = [-3, N, 2**31 - 1]
    y, am, av = w4.head_gather_tiled(tw, dev(x), row_ids=dev(ids), argmax=True)
    y, am, av = host(y), host(am), host(av)
    y_ref, a_ref = oracle.gather(ids, p, s, x)
    assert_parity(y, y_ref, a_ref, "tiled gather")
    for t in range(T):
        valid = ~np.isnan(y[t])
        best = np.max(y[t][valid])
        assert am[t] == ids[valid][y[t][valid] == best].min() and av[t] == best


@pytest.mark.parametrize("T", [1, 4])
def test_lm_head_tiled_argmax_and_draft_head(w4, T):
    n, k = synth.LM_HEAD
    p, s, pd, sd = weight_dev(synth.TID_LM_HEAD, n, k)
    tw = w4.repack_tiled(pd, sd)
    del pd, sd
    x = synth.activations(synth.TID_LM_HEAD + 7, T, k)
    say(f"tiled lm_head T={T}")
    y, am, _ = w4.head_gather_tiled(tw, dev(x), argmax=True)
    y, am = host(y), host(am)
    rows = sample_rows(n, 400, seed=T)
    y_ref, a_ref = oracle.gather(rows, p, s, x)
    assert_parity(y[:, rows], y_ref, a_ref, f"tiled lm_head T={T} (sampled)")
    own, _, _ = oracle.argmax(y.astype(np.float64))
    assert np.array_equal(am, own), "argmax differs from the argmax of the scores"
    # the oracle's argmax over all rows: equal unless a near-tie within the GPU's error
    full_ref, full_a = oracle.matmul(p, s, x)
    check_argmax(am, y, full_ref, None, f"tiled lm_head T={T}")
    if T == 1:
        ids = synth.distinct_ids(synth.RID_DRAFT, synth.DRAFT_IDS, n)
        yd, amd, _ = w4.head_gather_tiled(tw, dev(x), row_ids=dev(ids), argmax=True)
        yd, amd = host(yd), host(amd)
        assert np.array_equal(yd, y[:, ids]), "draft rows differ from the same rows of the full head"
        own_d, _, _ = oracle.argmax(yd.astype(np.float64), ids)
        assert np.array_equal(amd, own_d)


@pytest.mark.parametrize("T", [1, 5, 8])
def test_tall_tiled_below_head_size(w4, T):
    """A tall tiled matrix that one round of 16-wave runs would not fill
    (70,001 rows: 4,376 tiles) runs the 8-wave runs of 2 tiles: every score
    against the oracle, and its argmax, bit for bit against the host argmax
    of the scores and against the oracle's unless a near-tie."""
    N, K = 70001, 1024
    p, s, pd, sd = weight_dev(4500, N, K)
    tw = w4.repack_tiled(pd, sd)
    x = synth.activations(4500 + T, T, K)
    say(f"tall tiled {N}x{K} T={T}")
    y, am, av = w4.head_gather_tiled(tw, dev(x), argmax=True)
    y, am, av = host(y), host(am), host(av)
    y_ref, a_ref = oracle.matmul(p, s, x)
    assert_parity(y, y_ref, a_ref, f"tall tiled T={T}")
    own, _, _ = oracle.argmax(y.astype(np.float64))
    assert np.array_equal(am, own) and np.array_equal(av, y[np.arange(T), am])
    check_argmax(am, y, y_ref, None, f"tall tiled T={T}")
    assert np.array_equal(host(w4.matmul_tiled(tw, dev(x))), y), "matmul and head scores differ"


@pytest.mark.parametrize("N,K,T", [(16384, 5120, 8), (16400, 1024, 5), (32768, 2048, 6), (33000, 1024, 8),
                                   (100000, 1024, 7), (12301, 1152, 3), (14000, 17408, 2),
                                   # odd tile counts in 2-tile split workgroups
                                   (5121, 17408, 8), (7183, 5120, 1), (6001, 2304, 4)])
def test_mid_size_one_round_tilings(w4, N, K, T):
    """Mid-size and tall tiled matrices where the staging is dear take the
    one-round tilings (4, 8 or 16 waves of one tile; runs of 2 tiles per
    wave for 6,250 tiles), short ones from three quarters of a round at
    T >= 2 shared workgroups of 4 waves, and shorter ones from 1.25 tiles
    per CU split workgroups of 2 tiles (odd tile counts leave the last
    workgroup half empty): sampled rows against the oracle, including the
    tile edges."""
    p, s, pd, sd = weight_dev(4600 + T, N, K)
    tw = w4.repack_tiled(pd, sd)
    x = synth.activations(4600 + T, T, K)
    say(f"one-round tiling {N}x{K} T={T}")
    y = host(w4.matmul_tiled(tw, dev(x)))
    rows = sample_rows(N, 512, seed=N + T)
    y_ref, a_ref = oracle.gather(rows, p, s, x)
    assert_parity(y[:, rows], y_ref, a_ref, f"tiled {N}x{K} T={T}")


@pytest.mark.parametrize("T", [1, 4, 8])
def test_batch_mixed_layouts(w4, T):
    shapes = [(1024, 1024), (300, 5120), (17, 1152), (4099, 1280), (2000, 17408)]
    probs, host_side = [], []
    for i, (N, K) in enumerate(shapes):
        tid = 4400 + 10 * T + i
        p, s, pd, sd = weight_dev(tid, N, K)
        x = synth.activations(tid, T, K)
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        w = w4.repack_tiled(pd, sd) if i % 2 == 0 else pd
        probs.append((w, None if i % 2 == 0 else sd, dev(x), y))
        host_side.append((p, s, x))
    w4.Batch(probs, T).run()
    for (w, _, _, y), (p, s, x) in zip(probs, host_side):
        N = p.shape[0]
        rows = sample_rows(N, 256, seed=N) if N > 2048 else np.arange(N, dtype=np.int32)
        y_ref, a_ref = oracle.gather(rows, p, s, x)
        assert_parity(host(y)[:, rows], y_ref, a_ref, f"batch mixed T={T} N={N}")


@pytest.mark.parametrize("N,K,n_ids", [(300, 5120, 77), (37, 1152, 1), (1000, 2304, 2500)])
def test_repack_rows_matches_layout_of_gathered_rows(w4, N, K, n_ids):
    """The gathered repack is the layout of the host-gathered rows, byte for
    byte (duplicates included); an id outside [0, N) gives a row of zero
    codes whose scales are the bf16 quiet NaN 0x7FC0 (its scores are NaN)."""
    p, s, pd, sd = weight_dev(4300 + N + K, N, K)
    rng = np.random.default_rng(n_ids)
    ids = rng.integers(0, N, n_ids).astype(np.int32)
    ids[0] = N - 1
    tw = w4.repack_tiled_rows(pd, sd, dev(ids))
    assert tw.N == n_ids and tw.data.numel() == w4.tiled_bytes(n_ids, K)
    want = layout_by_definition(p[ids], s[ids])
    assert np.array_equal(host(tw.data), want)
    bad = ids.copy()
    bad[min(1, n_ids - 1)] = N + 5
    pz, sz = p[ids].copy(), s[ids].copy()
    pz[min(1, n_ids - 1)] = 0
    sz[min(1, n_ids - 1)] = 0x7FC0
    assert np.array_equal(host(w4.repack_tiled_rows(pd, sd, dev(bad)).data), layout_by_definition(pz, sz))


@pytest.mark.parametrize("T", [1, 4])
def test_compact_draft_head_matches_oracle(w4, T):
    """The 32,768-id draft head repacked once into its own tiled matrix:
    scores equal the oracle's gathered rows; the argmax position maps to the
    vocabulary id of the (ascending) id list and equals the host argmax."""
    from test_gpu_parity import lm_head

    p, s, pd, sd = lm_head()
    n_rows, K = synth.LM_HEAD
    ids = np.sort(synth.distinct_ids(synth.RID_DRAFT, synth.DRAFT_IDS, n_rows))
    x = synth.activations(synth.TID_LM_HEAD + 66, T, K)
    tw = w4.repack_tiled_rows(pd, sd, dev(ids))
    y, am, _ = w4.head_gather_tiled(tw, dev(x), scores=True, argmax=True)
    y, am = host(y), host(am)
    y_ref, a_ref = oracle.gather(ids, p, s, x)
    assert_parity(y, y_ref, a_ref, f"compact draft head T={T}")
    own, _, _ = oracle.argmax(y.astype(np.float64), ids)
    assert np.array_equal(ids[am], own)


def test_compact_head_bad_ids_never_win(w4):
    """A compact head (w4a16_repack_tiled_rows) whose list holds ids outside
    the head: those rows score NaN, so with every valid score negative the
    argmax is still the best valid row (an all-zero row scoring 0 would win)."""
    N, K, T = 3000, 1024, 2
    p = synth.codes(4600, N, K) & 0x77  # every code in 0..7: levels -8..-1
    s = synth.scales(4600, N, K)
    xf = np.abs(synth.bf16_to_f32(synth.activations(4600, T, K)).astype(np.float64)) + 0.25
    x = np.array([synth.bf16_from_double(v) for v in xf.ravel()], np.uint16).reshape(T, K)
    ids = synth.distinct_ids(4601, 700, N).copy()
    ids[[0, 5, 333, 699]] = [-3, N, N + 100, -(2 ** 31)]
    y_ref, a_ref = oracle.gather(ids, p, s, x)
    assert np.all(y_ref[~np.isnan(y_ref)] < 0)
    tw = w4.repack_tiled_rows(dev(p), dev(s), dev(ids))
    say("compact head with bad ids")
    y, am, av = w4.head_gather_tiled(tw, dev(x), argmax=True)
    y, am, av = host(y), host(am), host(av)
    assert np.array_equal(np.isnan(y), np.isnan(y_ref)), "bad-id rows must score NaN"
    assert_parity(y, y_ref, a_ref, "compact head with bad ids")
    check_argmax(am, y, y_ref, None, "compact head with bad ids")
    assert np.all(am >= 0) and np.all(ids[am] >= 0) and np.array_equal(av, y[np.arange(T), am])
