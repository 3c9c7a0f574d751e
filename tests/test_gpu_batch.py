"""GPU parity of the grouped launch (many matmuls in one kernel launch)."""
import os

import numpy as np
import pytest

import oracle
import synth
import contextlib

from gpu_util import assert_parity, batch_variant, dev, forced_tile, host, say, sample_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SHAPES = [(1024, 1024), (300, 5120), (17, 128), (4099, 1280), (2000, 17408), (7168, 5120)]


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    return w4a16


def build_case(T, seed0):
    probs, host_side = [], []
    for i, (N, K) in enumerate(SHAPES):
        tid = seed0 + i
        p, s = synth.weight(tid, N, K)
        x = synth.activations(tid, T, K)
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        probs.append((dev(p), dev(s), dev(x), y))
        host_side.append((p, s, x))
    return probs, host_side


def check_outputs(probs, host_side, what):
    for (pd, sd, xd, y), (p, s, x) in zip(probs, host_side):
        N = p.shape[0]
        rows = sample_rows(N, 256, seed=N) if N > 2048 else np.arange(N, dtype=np.int32)
        y_ref, a_ref = oracle.gather(rows, p, s, x)
        assert_parity(host(y)[:, rows], y_ref, a_ref, f"{what} N={N} K={p.shape[1] * 2}")


@pytest.mark.parametrize("tile", [None, "shared,1,4", "split,1,4", "split,4,2", "split,2,8", "shared,1,16", "run,2,8", "run,6,8", "run,3,16"])
@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_batch_matches_oracle(w4, tile, T):
    say(f"batch tile={tile} T={T}")
    probs, host_side = build_case(T, 600 + 10 * T)
    with forced_tile(w4, tile, batch=True) if tile else contextlib.nullcontext():
        b = w4.Batch(probs, T)
    if tile:  # the table runs the forced shape
        assert batch_variant(b) == {"split": 2, "shared": 3, "run": 4}[tile.split(",")[0]]
    b.run()
    check_outputs(probs, host_side, f"batch {tile} T={T}")
    first = [host(y).copy() for *_, y in probs]
    b.run()
    for f, (*_, y) in zip(first, probs):
        assert np.array_equal(f, host(y)), "second run differs"


@pytest.mark.parametrize("T", [3, 5, 6, 7, 8])
def test_batch_tiled_default_matches_oracle(w4, T):
    """The grouped launch's own tiling for tiled weights around the switch
    between four and six tiles per wave (eight-wave run workgroups; the
    17,408-column problem runs sliced shared workgroups in the same kernel)."""
    say(f"batch tiled default T={T}")
    probs, host_side = build_case(T, 650 + T)
    probs = [(w4.repack_tiled(pp, ss), None, xx, yy) for pp, ss, xx, yy in probs]
    w4.Batch(probs, T).run()
    check_outputs(probs, host_side, f"batch tiled T={T}")


def test_batch_equals_single_launch_within_tolerance(w4):
    T = 4
    probs, host_side = build_case(T, 700)
    w4.Batch(probs, T).run()
    for (pd, sd, xd, y), (p, s, x) in zip(probs, host_side):
        y1 = host(w4.matmul(pd, sd, xd))
        yb = host(y)
        # same arithmetic up to fp32 summation order
        y_ref, a_ref = oracle.matmul(p, s, x) if p.shape[0] <= 2048 else (None, None)
        if y_ref is not None:
            assert_parity(y1, y_ref, a_ref, "single")
            assert_parity(yb, y_ref, a_ref, "batch")


def test_batch_rejects_bad_tables(w4):
    lib = w4.load_library()
    junk = torch.zeros(256, dtype=torch.uint8)
    junk_dev = junk.cuda()
    assert lib.w4a16_matmul_batch(junk.data_ptr(), junk_dev.data_ptr(), None) == 2  # not a table


@pytest.mark.parametrize("T,tiled", [(1, True), (4, True), (8, True), (4, False), (16, True)])
def test_batch_with_lm_head_argmax(w4, T, tiled):
    """A verify pass in one grouped launch: some projections plus the full
    lm_head with its per-row argmax.  The head's scores equal a single
    head_gather launch's bit for bit (the same per-tile arithmetic), its
    argmax equals that launch's and the host argmax of the scores, and the
    other problems match the oracle."""
    from test_gpu_parity import lm_head

    say(f"batch + lm_head argmax T={T} tiled={tiled}")
    p, s, pd, sd = lm_head()
    n, k = synth.LM_HEAD
    x = dev(synth.activations(synth.TID_LM_HEAD + 60 + T, T, k))
    hw = w4.repack_tiled(pd, sd) if tiled else None
    probs, host_side = build_case(T, 800 + T)
    if tiled:
        probs = [(w4.repack_tiled(pp, ss), None, xx, yy) for pp, ss, xx, yy in probs]
    y = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
    am_id = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    am_val = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(w4.workspace_bytes(n, T), dtype=torch.uint8, device="cuda")
    head = (hw, None, x, y, am_id, am_val, ws) if tiled else (pd, sd, x, y, am_id, am_val, ws)
    b = w4.Batch(probs[:3] + [head] + probs[3:], T)
    b.run()
    if tiled:
        y1, i1, v1 = w4.head_gather_tiled(hw, x, scores=True, argmax=True)
    else:
        y1, i1, v1 = w4.head_gather(pd, sd, x, scores=True, argmax=True)
    yh = host(y)
    assert np.array_equal(yh, host(y1)), "scores differ from the single launch"
    assert np.array_equal(host(am_id), host(i1)) and np.array_equal(host(am_val), host(v1))
    own, _, _ = oracle.argmax(yh.astype(np.float64))
    assert np.array_equal(host(am_id), own)
    assert np.array_equal(host(am_val), yh[np.arange(T), host(am_id)])
    check_outputs([(None, None, None, yy) for *_, yy in probs], host_side, f"batch with head T={T}")
    # replay: the same ids again (the workspace holds no state between launches)
    am_id.fill_(-7)
    b.run()
    assert np.array_equal(host(am_id), host(i1))


@pytest.mark.parametrize("T", [9, 12, 16])
def test_batch_workspace_form_equals_plain_form(w4, T):
    """The workspace form of the grouped launch (w4a16_matmul_batch_ws) needs
    no workspace at any T and gives the plain launch's outputs bit for bit:
    rows scaled by 2^40 and 2^-40 and a row spanning 2^20, both layouts, a
    problem's argmax, all against the oracle."""
    say(f"workspace form T={T}")
    shapes = [(1000, 5120), (2000, 17408), (300, 1152), (17, 128)]
    probs, host_side = [], []
    for i, (N, K) in enumerate(shapes):
        tid = 900 + 10 * T + i
        p, s = synth.weight(tid, N, K)
        xf = synth.bf16_to_f32(synth.activations(tid, T, K)).astype(np.float64)
        xf[0] *= 2.0 ** 40
        xf[T - 1] *= 2.0 ** -40
        xf[T // 2, : K // 2] *= 2.0 ** -20
        x = np.array([synth.bf16_from_double(v) for v in xf.ravel()], np.uint16).reshape(T, K)
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        pd, sd = dev(p), dev(s)
        w = w4.repack_tiled(pd, sd) if i % 2 == 0 else pd
        probs.append((w, None if i % 2 == 0 else sd, dev(x), y))
        host_side.append((p, s, x))
    n_h = 1000
    am_id = torch.empty(T, dtype=torch.int32, device="cuda")
    am_val = torch.empty(T, dtype=torch.float32, device="cuda")
    ws = torch.empty(w4.workspace_bytes(n_h, T), dtype=torch.uint8, device="cuda")
    probs[0] = probs[0] + (am_id, am_val, ws)
    b = w4.Batch(probs, T)
    assert b.workspace is None
    lib = w4.load_library()
    st = lib.w4a16_matmul_batch_ws(b.host.data_ptr(), b.device.data_ptr(), None, 0,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, w4.status_string(st)
    with_ws = [host(pr[3]).copy() for pr in probs] + [host(am_id).copy(), host(am_val).copy()]
    for pr in probs:
        pr[3].fill_(-1.0)
    b.run()
    plain = [host(pr[3]).copy() for pr in probs] + [host(am_id).copy(), host(am_val).copy()]
    for i, (a_, b_) in enumerate(zip(with_ws, plain)):
        assert np.array_equal(a_, b_, equal_nan=True), f"output {i} differs between the two forms"
    check_outputs([(None, None, None, pr[3]) for pr in probs], host_side, f"grouped launch T={T}")
