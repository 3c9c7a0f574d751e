"""GPU parity for T = 9..16 activation rows in one weight read.

Several sequences with their drafts verified in one pass (the qwen-warp
article's outlook for several users: one weight read can serve as many as
16 activation rows, for instance 4 sequences carrying 3 drafts apiece).  Every case runs the
matrix-core kernels (the dot variant is built for T <= 8; selecting it at
larger T still runs the matrix cores), in both weight layouts, single and
grouped launches, and on the heads with argmax.  Expected values come only
from the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, dev, forced_tile, host, say, sample_rows, weight_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    w4a16.set_variant("auto")
    yield w4a16
    w4a16.set_variant("auto")


def both_layouts(w4, p, s, x):
    """(row-major result, tiled result) of one matmul."""
    pd, sd, xd = dev(p), dev(s), dev(x)
    y_rm = host(w4.matmul(pd, sd, xd))
    y_t = host(w4.matmul_tiled(w4.repack_tiled(pd, sd), xd))
    return y_rm, y_t


def test_small_matrix_t9_to_16(w4):
    N, K = synth.SMALL
    p, s = synth.weight(synth.TID_SMALL, N, K)
    for T in range(9, 17):
        say(f"small T={T}")
        x = synth.activations(synth.TID_SMALL + T, T, K)
        y_ref, a_ref = oracle.matmul(p, s, x)
        y_rm, y_t = both_layouts(w4, p, s, x)
        assert_parity(y_rm, y_ref, a_ref, f"small row-major T={T}")
        assert_parity(y_t, y_ref, a_ref, f"small tiled T={T}")


# single group; G = 9 (one scale per load); several activation slices
# (K = 17408); ragged tile tails; tall matrices for the run workgroups
RAGGED = [(1, 128, 16), (17, 384, 9), (33, 1152, 16), (4099, 1280, 12), (257, 5120, 16), (31, 17408, 16),
          (16400, 1024, 16), (17003, 1152, 11), (16413, 5120, 13)]


@pytest.mark.parametrize("N,K,T", RAGGED)
def test_ragged_shapes_t16(w4, N, K, T):
    say(f"ragged N={N} K={K} T={T}")
    tid = 5000 + N + K + T
    p, s = synth.weight(tid, N, K)
    x = synth.activations(tid, T, K)
    rows = sample_rows(N, 400, seed=tid) if N > 4096 else np.arange(N, dtype=np.int32)
    y_ref, a_ref = oracle.gather(rows, p, s, x)
    y_rm, y_t = both_layouts(w4, p, s, x)
    assert_parity(y_rm[:, rows], y_ref, a_ref, f"row-major N={N} K={K} T={T}")
    assert_parity(y_t[:, rows], y_ref, a_ref, f"tiled N={N} K={K} T={T}")


@pytest.mark.parametrize("proj", synth.PROJ_ORDER)
def test_projection_sampled_t16(w4, proj):
    """27B-class projections at T = 16: whole GPU output, oracle on sampled rows."""
    N, K = synth.PROJECTIONS[proj]
    tid = synth.tid_layer(1, proj)
    p, s = synth.weight(tid, N, K)
    x = synth.activations(tid, 16, K)
    rows = sample_rows(N, 192, seed=tid)
    y_ref, a_ref = oracle.gather(rows, p, s, x)
    y_rm, y_t = both_layouts(w4, p, s, x)
    assert np.all(np.isfinite(y_rm)) and np.all(np.isfinite(y_t))
    assert_parity(y_rm[:, rows], y_ref, a_ref, f"{proj} row-major T=16")
    assert_parity(y_t[:, rows], y_ref, a_ref, f"{proj} tiled T=16")


def test_single_level_rows_exact_t16(w4):
    """One code != 8 per row, every (k, q) at K = 128: bit-exact at T = 16."""
    K, T = 128, 16
    ks = np.repeat(np.arange(K), 16)
    qs = np.tile(np.arange(16), K)
    N = ks.size
    p = np.full((N, K // 2), 0x88, np.uint8)
    lo = ks % 2 == 0
    p[np.arange(N)[lo], ks[lo] // 2] = 0x80 | qs[lo]
    p[np.arange(N)[~lo], ks[~lo] // 2] = 0x08 | (qs[~lo] << 4)
    s = synth.scales(51, N, K)
    x = synth.activations(51, T, K)
    y_ref, _ = oracle.matmul(p, s, x)
    y_rm, y_t = both_layouts(w4, p, s, x)
    assert np.array_equal(y_rm.astype(np.float64), y_ref)
    assert np.array_equal(y_t.astype(np.float64), y_ref)


def test_all_eight_codes_zero_t16(w4):
    N, K, T = 100, 1152, 16
    p = np.full((N, K // 2), 0x88, np.uint8)
    s = synth.scales(52, N, K)
    y_rm, y_t = both_layouts(w4, p, s, synth.activations(52, T, K))
    assert np.all(y_rm == 0.0) and np.all(y_t == 0.0)


def test_extreme_activation_ranges_t16(w4):
    """Rows scaled by 2^40, 2^-40 and 2^20 among ordinary rows (scaled staging)."""
    N, K, T = 64, 1024, 16
    p, s = synth.weight(53, N, K)
    xf = synth.bf16_to_f32(synth.activations(53, T, K)).astype(np.float64)
    xf[0] *= 2.0 ** 40
    xf[9] *= 2.0 ** -40
    xf[15, :512] *= 2.0 ** 20
    x = np.array([synth.bf16_from_double(v) for v in xf.ravel()], np.uint16).reshape(T, K)
    y_ref, a_ref = oracle.matmul(p, s, x)
    y_rm, y_t = both_layouts(w4, p, s, x)
    assert_parity(y_rm, y_ref, a_ref, "extreme x row-major")
    assert_parity(y_t, y_ref, a_ref, "extreme x tiled")


def test_dot_selection_runs_matrix_cores_above_8(w4):
    N, K, T = 300, 1024, 12
    p, s = synth.weight(54, N, K)
    x = synth.activations(54, T, K)
    y_ref, a_ref = oracle.matmul(p, s, x)
    w4.set_variant("dot")
    try:
        y = host(w4.matmul(dev(p), dev(s), dev(x)))
    finally:
        w4.set_variant("auto")
    assert_parity(y, y_ref, a_ref, "dot selected at T=12")


@pytest.mark.parametrize("tile", ["split,1,8", "split,2,3", "shared,1,1", "shared,4,4", "shared,1,16", "run,3,4",
                                  "run,4,16"])
def test_tile_shapes_t16(w4, tile):
    with forced_tile(w4, tile):
        for N, K, T in [(37, 1152, 16), (300, 17408, 16), (4099, 5120, 14)]:
            say(f"tile {tile} N={N} K={K} T={T}")
            tid = 5200 + N + K + T
            p, s = synth.weight(tid, N, K)
            x = synth.activations(tid, T, K)
            rows = sample_rows(N, 300, seed=tid) if N > 2048 else np.arange(N, dtype=np.int32)
            y_ref, a_ref = oracle.gather(rows, p, s, x)
            y_rm, y_t = both_layouts(w4, p, s, x)
            assert_parity(y_rm[:, rows], y_ref, a_ref, f"{tile} row-major N={N} K={K} T={T}")
            assert_parity(y_t[:, rows], y_ref, a_ref, f"{tile} tiled N={N} K={K} T={T}")


@pytest.mark.parametrize("tiled", [True, False])
def test_batch_t16(w4, tiled):
    """Grouped launch of one layer's four projections (and two short ones) at T = 16."""
    T = 16
    shapes = [synth.PROJECTIONS[p] for p in synth.PROJ_ORDER] + [(300, 1152), (17, 128)]
    probs, host_side = [], []
    for i, (N, K) in enumerate(shapes):
        tid = 5400 + i
        p, s = synth.weight(tid, N, K)
        x = synth.activations(tid, T, K)
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        pd, sd = dev(p), dev(s)
        probs.append((w4.repack_tiled(pd, sd), None, dev(x), y) if tiled else (pd, sd, dev(x), y))
        host_side.append((p, s, x))
    w4.Batch(probs, T).run()
    for (_, _, _, y), (p, s, x) in zip(probs, host_side):
        N = p.shape[0]
        rows = sample_rows(N, 256, seed=N) if N > 2048 else np.arange(N, dtype=np.int32)
        y_ref, a_ref = oracle.gather(rows, p, s, x)
        assert_parity(host(y)[:, rows], y_ref, a_ref, f"batch T=16 N={N}")


def test_lm_head_argmax_t16(w4):
    """Full 248,320 x 5,120 head at T = 16 (tiled): every score vs the oracle,
    argmax equal to the host argmax of the GPU scores and to the oracle's
    (up to a near-tie narrower than the measured error)."""
    from gpu_util import check_argmax
    from test_gpu_parity import lm_head

    T = 16
    p, s, pd, sd = lm_head()
    x = synth.activations(synth.TID_LM_HEAD + 16, T, synth.LM_HEAD[1])
    say("oracle lm_head T=16 ...")
    y_ref, a_ref = oracle.matmul(p, s, x)
    tw = w4.repack_tiled(pd, sd)
    y, ids, vals = w4.head_gather_tiled(tw, dev(x), scores=True, argmax=True)
    y, ids, vals = host(y), host(ids), host(vals)
    assert_parity(y, y_ref, a_ref, "lm_head T=16")
    check_argmax(ids, y, y_ref, None, "lm_head T=16")
    assert np.array_equal(vals, y[np.arange(T), ids])
    y2, ids2, _ = w4.head_gather(pd, sd, dev(x), scores=True, argmax=True)
    assert_parity(host(y2), y_ref, a_ref, "lm_head row-major T=16")
    check_argmax(host(ids2), host(y2), y_ref, None, "lm_head row-major T=16")


def test_draft_head_t16(w4):
    from gpu_util import check_argmax
    from test_gpu_parity import lm_head

    T = 16
    p, s, pd, sd = lm_head()
    n_rows, K = synth.LM_HEAD
    ids = synth.distinct_ids(synth.RID_DRAFT, synth.DRAFT_IDS, n_rows)
    x = synth.activations(synth.TID_LM_HEAD + 17, T, K)
    y_ref, a_ref = oracle.gather(ids, p, s, x)
    y, am, _ = w4.head_gather_tiled(w4.repack_tiled(pd, sd), dev(x), row_ids=dev(ids), scores=True, argmax=True)
    y, am = host(y), host(am)
    assert_parity(y, y_ref, a_ref, "draft head T=16")
    check_argmax(am, y, y_ref, ids, "draft head T=16")


@pytest.mark.parametrize("T", [1, 8, 16])
def test_maximum_k(w4, T):
    """K = 2^20, the largest the ABI accepts (8,192 groups: hundreds of
    staged slices per wave), on a ragged 37-row matrix: every output against
    the oracle in both layouts, and with the dot variant where it applies."""
    N, K = 37, 1 << 20
    say(f"maximum K={K} T={T}")
    p, s = synth.weight(5600 + T, N, K)
    x = synth.activations(5600 + T, T, K)
    y_ref, a_ref = oracle.matmul(p, s, x)
    y_rm, y_t = both_layouts(w4, p, s, x)
    assert_parity(y_rm, y_ref, a_ref, f"max K row-major T={T}")
    assert_parity(y_t, y_ref, a_ref, f"max K tiled T={T}")
    if T <= 8:
        w4.set_variant("dot")
        try:
            y_dot = host(w4.matmul(dev(p), dev(s), dev(x)))
        finally:
            w4.set_variant("auto")
        assert_parity(y_dot, y_ref, a_ref, f"max K dot T={T}")
