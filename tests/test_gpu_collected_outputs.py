"""GPU parity of workgroups that collect their outputs in LDS.

A run workgroup (several whole tiles per wave) keeps its outputs in LDS
behind the staged activations and writes them token row by token row when
all its waves are done.  If all of K and the block do not fit its LDS
share together, on the tiled layout it stages K in slices that leave room
for the block and carries the partial sums there from slice to slice; in
the row-major kernels each tile's outputs are stored as the tile
completes.  These cases reach every side of that rule: ragged row counts
(the last workgroup's block clipped to n_out); K = 9,216 at T = 4
(activations and outputs fill an eight-wave workgroup's 80 KB exactly)
against K = 9,472 (the activations alone fill it); K = 8,192 at T = 8 in
sixteen-wave workgroups (160 KB exactly) against K = 8,320; K = 5,120 from
T = 13; T from 1 to 16 under the grouped launch's own run shapes and
forced ones; gathered rows with invalid ids (NaN outputs through the
block) with the argmax, the argmax without scores; a slice whose
activations miss every fp16 window (the exact bf16 loop) beside one that
keeps the fp16 form; a guard word after every output buffer to catch a
write past it.  Shared workgroups (every wave its own tiles over all of K)
of a grouped launch, from two token rows, pass their outputs through the
staging area once every wave is done, when it holds them: the grouped
cases also force shared shapes (one tile per wave, and four in the
row-major kernels).  Expected values come only from the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, check_argmax, dev, forced_tile, host, say, sample_rows, weight_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 7.0  # written after each output buffer; no kernel writes it


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    w4a16.set_variant("mfma")
    yield w4a16
    w4a16.set_variant("auto")


def guarded_output(T, N):
    """A NaN-filled [T][N] float32 tensor followed by 64 guard words."""
    buf = torch.full((T * N + 64,), float("nan"), dtype=torch.float32, device="cuda")
    buf[T * N:] = GUARD
    return buf, buf[:T * N].view(T, N)


def check_guard(buf, T, N, what):
    assert torch.all(buf[T * N:] == GUARD).item(), f"{what}: write past the outputs"


def rows_of(N, seed):
    return sample_rows(N, 256, seed=seed) if N > 2048 else np.arange(N, dtype=np.int32)


@pytest.mark.parametrize("tiled", [True, False])
@pytest.mark.parametrize("tile", [None, "run,4,8", "run,1,8", "run,3,16", "run,2,4", "shared,1,16", "shared,4,4"])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 9, 12, 13, 16])
def test_grouped_runs_collect_outputs(w4, tiled, tile, T):
    shapes = [(17, 128), (300, 5120), (1100, 1280), (4099, 1280), (2000, 9216), (700, 9472)]
    probs, refs, bufs = [], [], []
    for i, (N, K) in enumerate(shapes):
        tid = 9000 + 10 * i + T
        p, s, pd, sd = weight_dev(tid, N, K)
        x = synth.activations(tid, T, K)
        buf, y = guarded_output(T, N)
        w = (w4.repack_tiled(pd, sd), None) if tiled else (pd, sd)
        probs.append((*w, dev(x), y))
        rows = rows_of(N, tid)
        refs.append((rows, oracle.gather(rows, p, s, x)))
        bufs.append(buf)
    say(f"collected outputs grouped tiled={tiled} tile={tile} T={T}")
    with forced_tile(w4, tile, batch=True):
        b = w4.Batch(probs, T)
    b.run()
    for (N, K), prob, buf, (rows, (y_ref, a_ref)) in zip(shapes, probs, bufs, refs):
        what = f"grouped tiled={tiled} tile={tile} T={T} {N}x{K}"
        assert_parity(host(prob[3])[:, rows], y_ref, a_ref, what)
        check_guard(buf, T, N, what)


@pytest.mark.parametrize("N,K,T,tile", [(4099, 9216, 4, "run,4,8"), (4099, 9472, 4, "run,4,8"), (1003, 9216, 3, "run,4,8"),
                                        (300, 5120, 5, "run,4,8"), (37, 1152, 4, "run,4,8"), (2100, 8192, 8, "run,4,16"),
                                        (2100, 8320, 8, "run,4,16"), (700, 5120, 16, "run,4,16"), (700, 5120, 12, "run,3,16")])
def test_single_run_launch_at_the_lds_limit(w4, N, K, T, tile):
    tid = 9100 + N + K + T
    p, s, pd, sd = weight_dev(tid, N, K)
    x = synth.activations(tid, T, K)
    rows = rows_of(N, tid)
    y_ref, a_ref = oracle.gather(rows, p, s, x)
    tw = w4.repack_tiled(pd, sd)
    with forced_tile(w4, tile):
        for name, call in (("row-major", lambda out: w4.matmul(pd, sd, dev(x), out=out)),
                           ("tiled", lambda out: w4.matmul_tiled(tw, dev(x), out=out))):
            say(f"collected outputs single {name} N={N} K={K} T={T} tile={tile}")
            buf, y = guarded_output(T, N)
            call(y)
            assert_parity(host(y)[:, rows], y_ref, a_ref, f"single {name} N={N} K={K} T={T}")
            check_guard(buf, T, N, f"single {name} N={N} K={K} T={T}")


@pytest.mark.parametrize("T", [1, 2, 3, 4, 8])
def test_gathered_runs_bad_ids_and_argmax(w4, T):
    """NaN rows (invalid ids) pass through the collected block and never win
    the argmax; the argmax without scores takes the per-tile path."""
    N, K = 3000, 1280
    p, s, pd, sd = weight_dev(9200 + T, N, K)
    x = synth.activations(9200 + T, T, K)
    ids = np.random.default_rng(T).integers(0, N, 1999).astype(np.int32)
    ids[[0, 700, 1998]] = [-5, N, 2**31 - 1]
    tw = w4.repack_tiled(pd, sd)
    y_ref, a_ref = oracle.gather(ids, p, s, x)
    with forced_tile(w4, "run,2,8"):
        say(f"collected outputs gather T={T}")
        y, am, av = w4.head_gather_tiled(tw, dev(x), row_ids=dev(ids), scores=True, argmax=True)
        y, am, av = host(y), host(am), host(av)
        assert_parity(y, y_ref, a_ref, f"gather run T={T}")
        check_argmax(am, y, y_ref, ids, f"gather run T={T}")
        assert np.array_equal(av, np.nanmax(y, axis=1)), "argmax value is not the best score"
        _, am2, av2 = w4.head_gather_tiled(tw, dev(x), row_ids=dev(ids), scores=False, argmax=True)
        assert np.array_equal(host(am2), am) and np.array_equal(host(av2), av), "argmax without scores differs"


@pytest.mark.parametrize("T", [13, 16])
def test_sliced_runs_mixed_level_forms(w4, T):
    """K = 5,120 at T = 13 and 16 (tiled) runs in two slices; a value of
    2^-60 in group 2 of token row 0, some 75 binades below the row's largest
    values, leaves the first slice no fp16 window (bf16 levels) while the
    second keeps the fp16 form."""
    N, K = 1100, 5120
    tid = 9300 + T
    p, s, pd, sd = weight_dev(tid, N, K)
    x = synth.activations(tid, T, K).copy()
    x[0, 300] = 0x2180  # 2^-60
    rows = rows_of(N, tid)
    y_ref, a_ref = oracle.gather(rows, p, s, x)
    tw = w4.repack_tiled(pd, sd)
    say(f"sliced runs mixed forms single T={T}")
    buf, y = guarded_output(T, N)
    with forced_tile(w4, "run,4,16"):
        w4.matmul_tiled(tw, dev(x), out=y)
    assert_parity(host(y)[:, rows], y_ref, a_ref, f"sliced single T={T}")
    check_guard(buf, T, N, f"sliced single T={T}")
    say(f"sliced runs mixed forms grouped T={T}")
    buf2, y2 = guarded_output(T, N)
    w4.Batch([(tw, None, dev(x), y2)], T).run()
    assert_parity(host(y2)[:, rows], y_ref, a_ref, f"sliced grouped T={T}")
    check_guard(buf2, T, N, f"sliced grouped T={T}")
