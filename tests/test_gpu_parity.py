"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Inputs are seeded (synth); expected values come only from the oracle.  The
bar is |y_gpu - y_ref| <= 1e-3 * sum_k |w*x| + 1e-6 per element, exact
equality where every term is exactly representable, and bit-exact argmax ids
(except on a near-tie narrower than the GPU's measured error on the two rows).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, check_argmax, dev, host, say, sample_rows, weight_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

VARIANTS = ["mfma", "dot"]


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    yield w4a16
    w4a16.set_variant("auto")


def run_matmul(w4, variant, pd, sd, x):
    w4.set_variant(variant)
    return host(w4.matmul(pd, sd, dev(x)))


# ------------------------------------------------------------ small / ragged ----

@pytest.mark.parametrize("variant", VARIANTS)
def test_small_matrix_all_t(w4, variant):
    """1024 x 1024 (the small single-matmul workload), every T, full comparison."""
    N, K = synth.SMALL
    p, s, pd, sd = weight_dev(synth.TID_SMALL, N, K)
    for T in range(1, 9):
        say(f"small {variant} T={T}")
        x = synth.activations(synth.TID_SMALL, T, K)
        y_ref, a_ref = oracle.matmul(p, s, x)
        r = assert_parity(run_matmul(w4, variant, pd, sd, x), y_ref, a_ref, f"small T={T}")
        say(f"  max err/tol {r:.3g}")


RAGGED = [(1, 128, 1), (17, 384, 3), (33, 1152, 8), (100, 256, 5), (1003, 640, 2), (4099, 1280, 4),
          (257, 5120, 7), (31, 17408, 8), (2049, 128, 6),
          # tall enough for the streaming kernel: 8-group scale loads, and the
          # one-scale-per-load path (G = 9 groups, not a multiple of 8)
          (16400, 1024, 1), (17003, 1152, 3), (16413, 2304, 8),
          # short matrices near a round of 4-wave workgroups, and of 2-tile
          # split workgroups (row-major)
          (12301, 1152, 3), (5121, 2048, 1), (8191, 1280, 6)]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("N,K,T", RAGGED)
def test_ragged_shapes(w4, variant, N, K, T):
    say(f"ragged {variant} N={N} K={K} T={T}")
    tid = 100 + N + K + T
    p, s, pd, sd = weight_dev(tid, N, K)
    x = synth.activations(tid, T, K)
    y_ref, a_ref = oracle.matmul(p, s, x)
    assert_parity(run_matmul(w4, variant, pd, sd, x), y_ref, a_ref, f"N={N} K={K} T={T}")


# ------------------------------------------------------ full-size projections ----

@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("proj", synth.PROJ_ORDER)
def test_projection_sampled(w4, variant, proj):
    """27B-class projections at T = 1, 4, 8: whole GPU output, oracle on sampled rows."""
    N, K = synth.PROJECTIONS[proj]
    tid = synth.tid_layer(0, proj)
    p, s, pd, sd = weight_dev(tid, N, K)
    rows = sample_rows(N, 192, seed=tid)
    for T in (1, 4, 8):
        say(f"{proj} {variant} T={T}")
        x = synth.activations(tid, T, K)
        y = run_matmul(w4, variant, pd, sd, x)
        assert np.all(np.isfinite(y))
        y_ref, a_ref = oracle.gather(rows, p, s, x)
        r = assert_parity(y[:, rows], y_ref, a_ref, f"{proj} T={T}")
        say(f"  max err/tol {r:.3g}")


# ---------------------------------------------------------------- exactness ----

@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("K", [128, 256])
def test_single_level_rows_exact(w4, variant, K):
    """One code != 8 per row, every (k, q): y equals the exact product bit for bit."""
    T = 8
    ks = np.repeat(np.arange(K), 16)
    qs = np.tile(np.arange(16), K)
    N = ks.size
    p = np.full((N, K // 2), 0x88, np.uint8)
    lo = ks % 2 == 0
    p[np.arange(N)[lo], ks[lo] // 2] = 0x80 | qs[lo]
    p[np.arange(N)[~lo], ks[~lo] // 2] = 0x08 | (qs[~lo] << 4)
    s = synth.scales(41, N, K)
    x = synth.activations(41, T, K)
    y_ref, _ = oracle.matmul(p, s, x)
    y = run_matmul(w4, variant, dev(p), dev(s), x)
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("variant", VARIANTS)
def test_all_eight_codes_zero(w4, variant):
    N, K = 100, 1152
    p = np.full((N, K // 2), 0x88, np.uint8)
    s = synth.scales(42, N, K)
    for T in (1, 5, 8):
        y = run_matmul(w4, variant, dev(p), dev(s), synth.activations(42, T, K))
        assert np.all(y == 0.0)


def _scaled_bits(bits, c):
    f = synth.bf16_to_f32(bits).astype(np.float64) * c
    return np.array([synth.bf16_from_double(v) for v in f.ravel()], np.uint16).reshape(bits.shape)


@pytest.mark.parametrize("variant", VARIANTS)
def test_linearity_bitwise(w4, variant):
    N, K, T = 300, 2560, 4
    p, s, pd, sd = weight_dev(43, N, K)
    x = synth.activations(43, T, K)
    y = run_matmul(w4, variant, pd, sd, x)
    y_s2 = run_matmul(w4, variant, pd, dev(_scaled_bits(s, 2.0)), x)
    y_x2 = run_matmul(w4, variant, pd, sd, _scaled_bits(x, 2.0))
    y_xn = run_matmul(w4, variant, pd, sd, _scaled_bits(x, -1.0))
    # power-of-two factors commute with every fp32 rounding: bit-exact
    assert np.array_equal(y_s2, 2 * y)
    assert np.array_equal(y_x2, 2 * y)
    # negation: the matrix cores' internal fp32 sums are not sign-symmetric, so
    # -x is held to the tolerance, not to bitwise -y
    y_ref, a_ref = oracle.matmul(p, s, _scaled_bits(x, -1.0))
    assert_parity(y_xn, y_ref, a_ref, "negated x")
    assert_parity(-y, y_ref, a_ref, "negated y")


@pytest.mark.parametrize("variant", VARIANTS)
def test_rows_permute_bitwise_and_identical_rows(w4, variant):
    N, K, T = 512, 1280, 6
    p, s = synth.weight(44, N, K)
    p[300], s[300] = p[5], s[5]
    x = synth.activations(44, T, K)
    y = run_matmul(w4, variant, dev(p), dev(s), x)
    assert np.array_equal(y[:, 300], y[:, 5])
    perm = np.random.default_rng(1).permutation(N)
    yp = run_matmul(w4, variant, dev(p[perm]), dev(s[perm]), x)
    assert np.array_equal(yp, y[:, perm])


@pytest.mark.parametrize("variant", VARIANTS)
def test_misaligned_scale_rows(w4, variant):
    """Scales starting 2 bytes past a 16-byte boundary (allowed by the ABI)."""
    N, K, T = 16500, 1024, 4
    p, s = synth.weight(48, N, K)
    x = synth.activations(48, T, K)
    buf = torch.zeros(s.size + 8, dtype=torch.int16, device="cuda")
    sd = buf[1:1 + s.size].view(N, K // 128)
    sd.copy_(torch.from_numpy(s.view(np.int16)).cuda())
    assert sd.data_ptr() % 16 == 2
    y_ref, a_ref = oracle.matmul(p, s, x)
    assert_parity(run_matmul(w4, variant, dev(p), sd, x), y_ref, a_ref, "misaligned scales")


@pytest.mark.parametrize("variant", VARIANTS)
def test_extreme_activation_ranges(w4, variant):
    """Large and tiny activations still match (exact power-of-two staging)."""
    N, K, T = 64, 1024, 3
    p, s = synth.weight(45, N, K)
    xf = synth.bf16_to_f32(synth.activations(45, T, K)).astype(np.float64)
    xf[0] *= 2.0 ** 40
    xf[1] *= 2.0 ** -40
    xf[2, :512] *= 2.0 ** 20
    x = np.array([synth.bf16_from_double(v) for v in xf.ravel()], np.uint16).reshape(T, K)
    y_ref, a_ref = oracle.matmul(p, s, x)
    assert_parity(run_matmul(w4, variant, dev(p), dev(s), x), y_ref, a_ref, "extreme x")


# ------------------------------------------------------------ heads + argmax ----

_LM = {}


def lm_head():
    if "w" not in _LM:
        n, k = synth.LM_HEAD
        p, s = synth.weight(synth.TID_LM_HEAD, n, k)
        _LM["w"] = (p, s, dev(p), dev(s))
    return _LM["w"]


def lm_ref(T):
    if T not in _LM:
        p, s, _, _ = lm_head()
        x = synth.activations(synth.TID_LM_HEAD, T, synth.LM_HEAD[1])
        say(f"oracle lm_head T={T} ...")
        _LM[T] = (x,) + oracle.matmul(p, s, x)
    return _LM[T]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("T", [1, 4])
def test_lm_head_argmax(w4, variant, T):
    """Full 248,320 x 5,120 head: every score vs the oracle, argmax bit-exact."""
    p, s, pd, sd = lm_head()
    x, y_ref, a_ref = lm_ref(T)
    w4.set_variant(variant)
    say(f"lm_head {variant} T={T}")
    y, ids, vals = w4.head_gather(pd, sd, dev(x), scores=True, argmax=True)
    y, ids, vals = host(y), host(ids), host(vals)
    r = assert_parity(y, y_ref, a_ref, f"lm_head T={T}")
    say(f"  max err/tol {r:.3g}")
    check_argmax(ids, y, y_ref, None, f"lm_head T={T}")
    assert np.array_equal(vals, y[np.arange(T), ids])
    # argmax only (no score write) gives the same answer
    _, ids2, vals2 = w4.head_gather(pd, sd, dev(x), scores=False, argmax=True)
    assert np.array_equal(host(ids2), ids) and np.array_equal(host(vals2), vals)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("T", [1, 4])
def test_draft_head_gather(w4, variant, T):
    """32,768 draft-vocabulary rows gathered from the head."""
    p, s, pd, sd = lm_head()
    n_rows, K = synth.LM_HEAD
    ids = synth.distinct_ids(synth.RID_DRAFT, synth.DRAFT_IDS, n_rows)
    x = synth.activations(synth.TID_LM_HEAD + 7, T, K)
    y_ref, a_ref = oracle.gather(ids, p, s, x)
    w4.set_variant(variant)
    say(f"draft head {variant} T={T}")
    y, am, av = w4.head_gather(pd, sd, dev(x), row_ids=dev(ids), scores=True, argmax=True)
    y, am = host(y), host(am)
    assert_parity(y, y_ref, a_ref, f"draft head T={T}")
    check_argmax(am, y, y_ref, ids, f"draft head T={T}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_gather_identity_permutation_and_bad_ids(w4, variant):
    N, K, T = 3000, 1024, 4
    p, s, pd, sd = weight_dev(46, N, K)
    x = synth.activations(46, T, K)
    w4.set_variant(variant)
    y_full = host(w4.matmul(pd, sd, dev(x)))
    y_id, _, _ = w4.head_gather(pd, sd, dev(x))
    y_id = host(y_id)
    y_ref, a_ref = oracle.matmul(p, s, x)
    assert_parity(y_id, y_ref, a_ref, "identity gather")
    assert_parity(y_full, y_ref, a_ref, "matmul")
    perm = np.random.default_rng(2).permutation(N).astype(np.int32)
    y_p, _, _ = w4.head_gather(pd, sd, dev(x), row_ids=dev(perm))
    y_p2, _, _ = w4.head_gather(pd, sd, dev(x), row_ids=dev(np.arange(N, dtype=np.int32)))
    assert np.array_equal(host(y_p), host(y_p2)[:, perm])
    bad = np.array([5, -1, N, 17, 2**31 - 1, 5], np.int32)
    y_b, am, av = w4.head_gather(pd, sd, dev(x), row_ids=dev(bad), argmax=True)
    y_b, am = host(y_b), host(am)
    assert np.all(np.isnan(y_b[:, [1, 2, 4]])) and not np.any(np.isnan(y_b[:, [0, 3, 5]]))
    yg_ref, ag_ref = oracle.gather(bad, p, s, x)
    assert_parity(y_b, yg_ref, ag_ref, "gather with bad ids")
    assert np.array_equal(y_b[:, 0], y_b[:, 5])
    check_argmax(am, y_b, yg_ref, bad, "bad ids")


@pytest.mark.parametrize("variant", VARIANTS)
def test_argmax_ties_and_no_valid_row(w4, variant):
    N, K, T = 700, 512, 2
    p, s = synth.weight(47, N, K)
    x = synth.activations(47, T, K)
    xf = synth.bf16_to_f32(x)[0]
    lev = np.where(xf > 0, 15, 0).astype(np.uint8)
    p[123] = lev[0::2] | (lev[1::2] << 4)
    s[123] = synth.bf16_from_double(0.5)
    p[650], s[650] = p[123], s[123]   # exact tie at a higher id
    w4.set_variant(variant)
    _, am, av = w4.head_gather(dev(p), dev(s), dev(x), argmax=True, scores=False)
    assert host(am)[0] == 123
    # gathered in reverse order: the lower vocabulary id still wins
    ids = np.arange(N - 1, -1, -1, dtype=np.int32)
    _, am2, _ = w4.head_gather(dev(p), dev(s), dev(x), row_ids=dev(ids), argmax=True, scores=False)
    assert host(am2)[0] == 123
    # no valid row at all
    _, am3, av3 = w4.head_gather(dev(p), dev(s), dev(x), row_ids=dev(np.array([-5, N, N + 1], np.int32)),
                                 argmax=True, scores=False)
    assert host(am3).tolist() == [-1, -1] and np.all(np.isnan(host(av3)))
