"""GPU parity of the verify epilogue: per-row top-k of head scores and greedy
acceptance, through the C ABI, against the oracle.

Selection is index work, so the bar is bit-exact: the GPU's top-k of a score
array equals the oracle's top-k of the same fp32 scores, ids and values.
Against the oracle's own scores the j-th largest value may move by at most
the largest per-element error (an order statistic is 1-Lipschitz in the max
norm), and ids must agree wherever the oracle's neighbouring values are
further apart than twice that error.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, host, say, tolerance

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    return w4a16


def check_topk_exact(w4, y, k, ids=None, what=""):
    """GPU top-k of y (float32 [T][n]) == oracle top-k of the same values."""
    y = np.ascontiguousarray(y, np.float32)
    got_id, got_val = w4.topk(dev(y), k, row_ids=None if ids is None else dev(ids))
    got_id, got_val = host(got_id), host(got_val)
    ref_id, ref_val = oracle.topk(y.astype(np.float64), k, ids)
    assert np.array_equal(got_id, ref_id), f"{what}: ids differ\n{got_id}\n{ref_id}"
    assert np.array_equal(got_val.astype(np.float64), ref_val, equal_nan=True), f"{what}: values differ"
    return got_id, got_val


@pytest.mark.parametrize("T,n,k", [(1, 1, 1), (1, 5, 32), (2, 2047, 7), (3, 2048, 32), (4, 2049, 32), (16, 10000, 16),
                                   (5, 123457, 32), (1, 3_000_000, 32)])
def test_topk_random_with_ties_and_nans(w4, T, n, k):
    say(f"topk T={T} n={n} k={k}")
    rng = np.random.default_rng(n + k)
    y = (np.round(rng.normal(size=(T, n)) * 4) / 4).astype(np.float32)  # many exact ties
    y[rng.random((T, n)) < 0.05] = np.nan
    y[:, rng.integers(0, n, size=min(n, 3))] = -0.0
    check_topk_exact(w4, y, k, what=f"T={T} n={n} k={k}")


def test_topk_gathered_ids_negative_ids_and_all_nan(w4):
    rng = np.random.default_rng(7)
    T, n, k = 3, 5000, 32
    y = rng.normal(size=(T, n)).astype(np.float32)
    ids = rng.permutation(400_000)[:n].astype(np.int32)
    ids[[4, 99, 4000]] = [-1, -7, -2**31]      # never counted, even with a finite score
    y[2, :] = np.nan                         # a row with nothing to count
    y[1, 10:20] = y[1, 10]                   # ten-way tie: ascending vocabulary ids
    got_id, got_val = check_topk_exact(w4, y, k, ids, "gathered")
    assert np.all(got_id[2] == -1) and np.all(np.isnan(got_val[2]))


def test_topk_fallback_paths(w4):
    """Both sort fallbacks: duplicated (id, score) keys fill a chunk's
    candidate list (chunk sort); ascending scores put every top chunk list
    above the bound (row merge by sorting)."""
    n = 5000
    y = np.full((2, n), 1.5, np.float32)
    ids = np.full(n, 77, np.int32)
    ids[4321] = 12                                        # one lower id with the same score
    check_topk_exact(w4, y, 32, ids, "duplicated keys")
    y = np.tile(np.arange(100_000, dtype=np.float32), (3, 1))
    y[1] *= -1.0                                          # and descending
    y[2, ::7] = np.nan
    check_topk_exact(w4, y, 32, what="monotone scores")
    check_topk_exact(w4, y, 5, what="monotone scores k=5")


def test_topk_of_the_lm_head_t4(w4):
    """k = 32 of the full 248,320-row head: exact on the GPU's scores, entry 0
    equal to the head kernel's argmax, and stable against the oracle's scores."""
    from test_gpu_parity import lm_head, lm_ref

    T, k = 4, 32
    p, s, pd, sd = lm_head()
    x, y_ref, a_ref = lm_ref(T)
    y, am, av = w4.head_gather(pd, sd, dev(x), scores=True, argmax=True)
    got_id, got_val = check_topk_exact(w4, host(y), k, what="lm_head")
    assert np.array_equal(got_id[:, 0], host(am)) and np.array_equal(got_val[:, 0], host(av))
    yg = host(y).astype(np.float64)
    ref_id, ref_val = oracle.topk(y_ref, k)
    for t in range(T):
        err = np.max(np.abs(yg[t] - y_ref[t]))
        assert err <= np.max(tolerance(a_ref[t]))
        assert np.all(np.abs(got_val[t].astype(np.float64) - ref_val[t]) <= err + 1e-30)
        v = ref_val[t]
        gaps = np.minimum(np.append(np.inf, v[:-1] - v[1:]), np.append(v[:-1] - v[1:], np.inf))
        clear = gaps > 2 * err
        assert np.array_equal(got_id[t][clear], ref_id[t][clear]), f"t={t}"
        say(f"  t={t}: max err {err:.3g}, {int(clear.sum())}/{k} positions separated")


def test_topk_of_the_draft_head_t16(w4):
    from test_gpu_parity import lm_head

    T, k = 16, 32
    p, s, pd, sd = lm_head()
    ids = synth.distinct_ids(synth.RID_DRAFT, synth.DRAFT_IDS, synth.LM_HEAD[0])
    x = synth.activations(synth.TID_LM_HEAD + 33, T, synth.LM_HEAD[1])
    y, am, _ = w4.head_gather(pd, sd, dev(x), row_ids=dev(ids), scores=True, argmax=True)
    got_id, _ = check_topk_exact(w4, host(y), k, ids, "draft head")
    assert np.array_equal(got_id[:, 0], host(am))


@pytest.mark.parametrize("rows", [1, 2, 4, 8, 16])
def test_greedy_accept_matches_oracle(w4, rows):
    rng = np.random.default_rng(rows)
    S = 1000
    target = rng.integers(0, 5, size=(S, rows)).astype(np.int32)
    target[rng.random((S, rows)) < 0.02] = -1
    draft = np.where(rng.random((S, max(rows - 1, 0))) < 0.8, target[:, :rows - 1],
                     rng.integers(0, 5, size=(S, max(rows - 1, 0)))).astype(np.int32)
    acc, tok = w4.greedy_accept(dev(target.ravel()), dev(draft.ravel()) if rows > 1 else None, S, rows)
    ref_acc, ref_tok = oracle.greedy_accept(target.ravel(), draft.ravel(), S, rows)
    assert np.array_equal(host(acc), ref_acc) and np.array_equal(host(tok), ref_tok)


def test_verify_cycle_four_sequences_of_four_rows(w4):
    """T = 16 rows = 4 sequences x (1 + 3 drafts) in one head pass: the GPU's
    argmax ids feed the GPU acceptance; the oracle's chain on the GPU scores
    gives the same accepted counts and tokens."""
    from test_gpu_parity import lm_head

    S, L = 4, 4
    p, s, pd, sd = lm_head()
    x = synth.activations(synth.TID_LM_HEAD + 44, S * L, synth.LM_HEAD[1])
    y, am, _ = w4.head_gather(pd, sd, dev(x), scores=True, argmax=True)
    am_h = host(am)
    # drafts: sequence s agrees with the target for its first s rows, then differs
    draft = np.empty((S, L - 1), np.int32)
    for q in range(S):
        for j in range(L - 1):
            tgt = am_h[q * L + j]
            draft[q, j] = tgt if j < q else (tgt + 1) % synth.LM_HEAD[0]
    acc, tok = w4.greedy_accept(am, dev(draft.ravel()), S, L)
    own_id, _, _ = oracle.argmax(host(y).astype(np.float64))
    ref_acc, ref_tok = oracle.greedy_accept(own_id, draft.ravel(), S, L)
    assert np.array_equal(host(acc), ref_acc) and np.array_equal(host(tok), ref_tok)
    assert host(acc).tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("n_base,n_seq,n_rows", [(32768, 4096, 248320), (0, 10, 100), (5, 0, 100), (1, 4096, 524288),
                                                 (1000, 1, 1000), (3, 4000, 17)])
def test_draft_union_matches_oracle(w4, n_base, n_seq, n_rows):
    say(f"draft union base={n_base} seq={n_seq} vocab={n_rows}")
    rng = np.random.default_rng(n_base + n_seq)
    base = synth.distinct_ids(synth.RID_DRAFT + 1, n_base, n_rows) if n_base else np.empty(0, np.int32)
    pick = rng.random(n_seq)
    seq = np.where(pick < 0.4, rng.integers(0, n_rows, n_seq),                           # anywhere
                   np.where(pick < 0.7, base[rng.integers(0, max(n_base, 1), n_seq)] if n_base
                            else rng.integers(0, n_rows, n_seq),                          # in the base list
                            rng.integers(-5, n_rows + 5, n_seq))).astype(np.int32)        # some out of range
    if n_seq > 8:
        seq[n_seq // 2:n_seq // 2 + 4] = seq[1]                                           # repeats
    ids, length = w4.draft_union(dev(base) if n_base else None, dev(seq) if n_seq else None, n_rows)
    ref, m = oracle.draft_union(base, seq, n_rows)
    assert np.array_equal(host(ids), ref) and int(host(length)[0]) == m


def test_draft_head_with_sequence_tokens(w4):
    """Union list -> one gathered pass over the full head (capacity n_base +
    n_seq rows): the listed rows match the oracle, the -1 slots are NaN, and
    argmax and top-k count only listed rows."""
    from test_gpu_parity import lm_head

    T, k = 4, 32
    p, s, pd, sd = lm_head()
    n_rows, K = synth.LM_HEAD
    base = synth.distinct_ids(synth.RID_DRAFT, synth.DRAFT_IDS, n_rows)
    rng = np.random.default_rng(99)
    seq = np.concatenate([base[rng.integers(0, base.size, 300)], rng.integers(0, n_rows, 700)]).astype(np.int32)
    ids_d, length = w4.draft_union(dev(base), dev(seq), n_rows)
    ids = host(ids_d)
    m = int(host(length)[0])
    x = synth.activations(synth.TID_LM_HEAD + 55, T, K)
    y, am, av = w4.head_gather_tiled(w4.repack_tiled(pd, sd), dev(x), row_ids=ids_d, scores=True, argmax=True)
    y, am = host(y), host(am)
    assert np.all(np.isnan(y[:, m:])) and not np.any(np.isnan(y[:, :m]))
    rows = np.concatenate([np.arange(0, m, 97), np.arange(synth.DRAFT_IDS - 3, m)]).astype(np.int64)
    y_ref, a_ref = oracle.gather(ids[rows], p, s, x)
    from gpu_util import assert_parity
    assert_parity(y[:, rows], y_ref, a_ref, "draft head with sequence tokens")
    own, _, _ = oracle.argmax(y.astype(np.float64), ids)
    assert np.array_equal(am, own)
    check_topk_exact(w4, y, k, ids, "union top-k")
