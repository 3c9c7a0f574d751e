"""The allocation-free head call, w4a16_head_gather_noalloc, through the C
ABI: every output equal bit for bit to w4a16_head_gather's (the same
kernels, the argmax partials in the library's static scratch instead of the
caller's workspace) and within the oracle's tolerance, on two calls in a
row whose second is smaller (the scratch keeps the first call's contents),
one of them at the scratch's size limit, and a call beyond the limit
refused with nothing written."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, check_argmax, dev, host, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCRATCH_STATUS = 8


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    return w4a16


def noalloc(lib, pd, sd, xd, ids, n_ids, n_rows, K, T, y, am, av):
    stream = torch.cuda.current_stream().cuda_stream
    return lib.w4a16_head_gather_noalloc(None if ids is None else ids.data_ptr(), n_ids, pd.data_ptr(),
                                         sd.data_ptr(), n_rows, xd.data_ptr(), K, T,
                                         None if y is None else y.data_ptr(), am.data_ptr(), av.data_ptr(), stream)


@pytest.mark.parametrize("variant", ["mfma", "dot"])
def test_noalloc_equals_workspace_call(w4, variant):
    lib = w4.load_library()
    w4.set_variant(variant)
    try:
        # the first call fills the scratch to its limit (262,144 rows at T = 16:
        # exactly W4A16_NOALLOC_SCRATCH_BYTES of partials; the dot variant is
        # built for T <= 8 and the call runs the matrix cores there), the second
        # is smaller and gathers rows with bad ids
        cases = [(262144, 128, 16, None), (9000, 5120, 4, 3100), (700, 1024, 1, 500)]
        for N, K, T, n_ids in cases:
            tid = 8100 + N + K + T
            p, s = synth.weight(tid, N, K)
            x = synth.activations(tid, T, K)
            pd, sd, xd = dev(p), dev(s), dev(x)
            if n_ids is None:
                ids_h, ids, n = None, None, N
            else:
                ids_h = synth.distinct_ids(tid, n_ids, N).copy()
                ids_h[[1, n_ids // 2]] = [-1, N + 3]
                ids, n = dev(ids_h), n_ids
            say(f"noalloc {variant} N={N} K={K} T={T} n={n}")
            y_ws, am_ws, av_ws = w4.head_gather(pd, sd, xd, row_ids=ids, argmax=True)
            y = torch.full((T, n), float("nan"), dtype=torch.float32, device="cuda")
            am = torch.full((T,), -7, dtype=torch.int32, device="cuda")
            av = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
            st = noalloc(lib, pd, sd, xd, ids, n, N, K, T, y, am, av)
            assert st == 0, w4.status_string(st)
            y_h, am_h, av_h = host(y), host(am), host(av)
            assert np.array_equal(y_h, host(y_ws), equal_nan=True), "scores differ from the workspace call"
            assert np.array_equal(am_h, host(am_ws)) and np.array_equal(av_h, host(av_ws), equal_nan=True)
            # the argmax alone (no scores): the same ids again
            am.fill_(-7)
            av.fill_(7.0)
            assert noalloc(lib, pd, sd, xd, ids, n, N, K, T, None, am, av) == 0
            assert np.array_equal(host(am), am_h) and np.array_equal(host(av), av_h, equal_nan=True)
            # against the oracle
            y_ref, a_ref = oracle.gather(ids_h if ids_h is not None else np.arange(N, dtype=np.int32), p, s, x)
            assert_parity(y_h, y_ref, a_ref, f"noalloc N={N} T={T}")
            check_argmax(am_h, y_h, y_ref, ids_h, f"noalloc N={N} T={T}")
    finally:
        w4.set_variant("auto")


def test_noalloc_refuses_beyond_its_scratch(w4):
    lib = w4.load_library()
    N, K, T = 262145, 128, 16
    p, s = synth.weight(8200, N, K)
    x = synth.activations(8200, T, K)
    pd, sd, xd = dev(p), dev(s), dev(x)
    y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    am = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    av = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
    assert noalloc(lib, pd, sd, xd, None, N, N, K, T, y, am, av) == SCRATCH_STATUS
    torch.cuda.synchronize()
    assert np.all(np.isnan(host(y))) and np.all(host(am) == -7), "a refused call must write nothing"
    # without the argmax the scratch is not used: the same shape runs
    st = lib.w4a16_head_gather_noalloc(None, N, pd.data_ptr(), sd.data_ptr(), N, xd.data_ptr(), K, T, y.data_ptr(),
                                       None, None, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    rows = np.array([0, 1, N // 2, N - 2, N - 1], np.int32)
    y_ref, a_ref = oracle.gather(rows, p, s, x)
    assert_parity(host(y)[:, rows], y_ref, a_ref, "noalloc without argmax")
