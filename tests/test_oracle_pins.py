"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something it does not compute itself: the
article's exhaustive nibble check, hand-computed examples, closed forms for
inputs with a single non-zero level, exact invariants (zero point, linearity,
row permutation) and brute-force argmax on tiny inputs.  A plausible slip in
the oracle -- swapped nibble order, a group boundary off by one, a missing
zero point, a sign error, a transposed operand, a wrong tie-break -- makes at
least one of them fail (see the planted-mistake tests at the end).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf16_bits(v: float) -> int:
    b = synth.bf16_from_double(v)
    assert synth.bf16_to_f32(np.array([b], np.uint16))[0] == np.float32(v), f"{v} not exact in bf16"
    return b


def fill_bf16(shape, v):
    return np.full(shape, bf16_bits(v), np.uint16)


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- levels ----

def test_bf16_constants_of_the_article():
    g = load("nibble_levels.json")
    assert oracle.bf16(int(g["bf16_128"], 16)) == 128.0
    assert oracle.bf16(int(g["bf16_one"], 16)) == 1.0
    assert oracle.bf16(int(g["bf16_minus_136"], 16)) == -136.0


def test_every_code_lands_on_its_level():
    """Article: (0x4300 | q) * 1.0 - 136 is exactly q - 8 for all sixteen codes."""
    g = load("nibble_levels.json")
    for q, level in zip(g["codes"], g["levels"]):
        # the article's bit identity, evaluated on the host
        assert oracle.bf16(0x4300 | q) * 1.0 - 136.0 == level
        # the oracle's own dequantisation of a lone code q at k=0 (x=1, s=1)
        packed = np.full((1, 64), 0x88, np.uint8)
        packed[0, 0] = 0x80 | q
        y, a = oracle.matmul(packed, fill_bf16((1, 1), 1.0), np.concatenate(
            [fill_bf16((1, 1), 1.0), fill_bf16((1, 127), 0.0)], axis=1))
        assert y[0, 0] == level and a[0, 0] == abs(level)


def test_code_extraction_per_byte():
    row = np.array([0x21, 0x43, 0xFE], np.uint8)
    assert [oracle.code(row, k) for k in range(6)] == [1, 2, 3, 4, 0xE, 0xF]


# ---------------------------------------------------------- hand examples ----

def test_hand_example_nibble_order():
    g = load("hand_examples.json")["H1_nibble_order"]
    packed = np.empty((2, 128), np.uint8)
    packed[0] = 0x99
    packed[1] = 0x0F
    scales = np.array([[bf16_bits(v) for v in r] for r in g["scales"]], np.uint16)
    x = np.empty((2, 256), np.uint16)
    x[0] = bf16_bits(1.0)
    x[1, 0::2] = bf16_bits(1.0)
    x[1, 1::2] = bf16_bits(0.0)
    y, _ = oracle.matmul(packed, scales, x)
    assert y.tolist() == g["y"]
    y2 = oracle.matmul_dequant_first(packed, scales, x)
    assert y2.tolist() == g["y"]


def test_hand_example_group_boundary():
    g = load("hand_examples.json")["H2_group_boundary"]
    packed = np.full((1, 128), 0x88, np.uint8)
    packed[0, 63] = 0xF8
    packed[0, 64] = 0x80
    scales = np.array([[bf16_bits(v) for v in g["scales"]]], np.uint16)
    y, _ = oracle.matmul(packed, scales, fill_bf16((1, 256), 1.0))
    assert y[0, 0] == g["y"]


# ------------------------------------------------------------ closed forms ----

@pytest.mark.parametrize("K", [128, 256])
def test_single_level_closed_form(K):
    """Rows with one code != 8: y = (q-8) * s * x_k exactly, for every (k, q)."""
    T = 8
    ks = np.repeat(np.arange(K), 16)
    qs = np.tile(np.arange(16), K)
    N = ks.size
    packed = np.full((N, K // 2), 0x88, np.uint8)
    for n, (k, q) in enumerate(zip(ks, qs)):
        b = packed[n, k // 2]
        packed[n, k // 2] = (b & 0xF0) | q if k % 2 == 0 else (b & 0x0F) | (q << 4)
    scales = synth.scales(11, N, K)
    x = synth.activations(11, T, K)
    y, a = oracle.matmul(packed, scales, x)
    s = synth.bf16_to_f32(scales).astype(np.float64)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    expect = (qs - 8)[None, :] * s[np.arange(N), ks // 128][None, :] * xf[:, ks]
    assert np.array_equal(y, expect)
    assert np.array_equal(a, np.abs(expect))


def test_all_eight_codes_give_zero():
    packed = np.full((16, 512), 0x88, np.uint8)
    y, a = oracle.matmul(packed, synth.scales(12, 16, 1024), synth.activations(12, 8, 1024))
    assert np.all(y == 0.0) and np.all(a == 0.0)


# -------------------------------------------------------------- invariants ----

def _case(seed_tid, N=24, K=384, T=5):
    p, s = synth.weight(seed_tid, N, K)
    return p, s, synth.activations(seed_tid, T, K)


def _times(bits, c):
    f = synth.bf16_to_f32(bits).astype(np.float64) * c
    out = np.array([synth.bf16_from_double(v) for v in f.ravel()], np.uint16).reshape(bits.shape)
    assert np.array_equal(synth.bf16_to_f32(out).astype(np.float64), f), "scaled value not exact in bf16"
    return out


def test_linearity_power_of_two_is_exact():
    p, s, x = _case(21)
    y, _ = oracle.matmul(p, s, x)
    y_s2, _ = oracle.matmul(p, _times(s, 2.0), x)
    y_x2, _ = oracle.matmul(p, s, _times(x, 2.0))
    y_xn, _ = oracle.matmul(p, s, _times(x, -1.0))
    assert np.array_equal(y_s2, 2 * y)
    assert np.array_equal(y_x2, 2 * y)
    assert np.array_equal(y_xn, -y)


def test_linearity_general_scale_factor():
    p, s, x = _case(22)
    y, a = oracle.matmul(p, s, x)
    # 1.5 keeps a scale exact in bf16 when its last two mantissa bits are 0 (6 + 2 significant bits)
    sf = synth.bf16_to_f32(s).astype(np.float64)
    s_even = np.array([synth.bf16_from_double(v) for v in sf.ravel()], np.uint16).reshape(s.shape) & 0xFFFC
    y0, a0 = oracle.matmul(p, s_even, x)
    y1, _ = oracle.matmul(p, _times(s_even, 1.5), x)
    assert np.all(np.abs(y1 - 1.5 * y0) <= 1e-12 * a0 + 1e-300)


def test_row_permutation_permutes_output():
    p, s, x = _case(23)
    perm = np.random.default_rng(0).permutation(p.shape[0])
    y, _ = oracle.matmul(p, s, x)
    yp, _ = oracle.matmul(p[perm], s[perm], x)
    assert np.array_equal(yp, y[:, perm])


def test_identical_rows_identical_values():
    p, s, x = _case(24)
    p[7] = p[3]
    s[7] = s[3]
    y, _ = oracle.matmul(p, s, x)
    assert np.array_equal(y[:, 7], y[:, 3])


def test_two_forms_agree():
    for tid, (N, K, T) in enumerate([(3, 128, 1), (17, 640, 4), (33, 1280, 8)]):
        p, s = synth.weight(30 + tid, N, K)
        x = synth.activations(30 + tid, T, K)
        y, a = oracle.matmul(p, s, x)
        y2 = oracle.matmul_dequant_first(p, s, x)
        assert np.all(np.abs(y - y2) <= 1e-12 * a)


def test_summation_error_within_double_bound():
    """The only rounding is the sum: compare with exact summation (math.fsum)."""
    p, s, x = _case(25, N=6, K=1024, T=2)
    y, a = oracle.matmul(p, s, x)
    sf = synth.bf16_to_f32(s).astype(np.float64)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    lo = (p & 0x0F).astype(np.int64) - 8
    hi = (p >> 4).astype(np.int64) - 8
    lev = np.empty((p.shape[0], 1024), np.int64)
    lev[:, 0::2], lev[:, 1::2] = lo, hi
    w = lev * np.repeat(sf, 128, axis=1)
    for t in range(2):
        for n in range(6):
            exact = math.fsum(w[n] * xf[t])
            assert abs(y[t, n] - exact) <= 1024 * 2.0**-53 * a[t, n]


def test_threads_do_not_change_results():
    p, s, x = _case(26, N=40)
    y1, a1 = oracle.matmul(p, s, x, nthreads=1)
    y8, a8 = oracle.matmul(p, s, x, nthreads=8)
    assert np.array_equal(y1, y8) and np.array_equal(a1, a8)


# ------------------------------------------------------------------ gather ----

def test_gather_equals_rows_of_full_matrix():
    p, s, x = _case(27, N=50)
    y, a = oracle.matmul(p, s, x)
    ids = np.array([49, 0, 7, 7, 23], np.int32)
    yg, ag = oracle.gather(ids, p, s, x)
    assert np.array_equal(yg, y[:, ids]) and np.array_equal(ag, a[:, ids])


def test_gather_out_of_range_is_nan():
    p, s, x = _case(28, N=10)
    yg, _ = oracle.gather(np.array([3, -1, 10, 9], np.int32), p, s, x)
    assert np.all(np.isnan(yg[:, 1])) and np.all(np.isnan(yg[:, 2]))
    assert not np.any(np.isnan(yg[:, [0, 3]]))


# ------------------------------------------------------------------ argmax ----

def brute_argmax(values, ids):
    cand = [(v, i) for v, i in zip(values, ids) if not math.isnan(v)]
    if not cand:
        return -1
    best = max(v for v, _ in cand)
    return min(i for v, i in cand if v == best)


def test_argmax_brute_force_tiny():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        vals = rng.integers(-3, 4, size=(3, n)).astype(np.float64)  # many ties
        vals[rng.random((3, n)) < 0.2] = np.nan
        ids = rng.permutation(100)[:n].astype(np.int32)
        got, val, _ = oracle.argmax(vals, ids)
        for t in range(3):
            assert got[t] == brute_argmax(vals[t], ids.tolist())
        got_pos, _, _ = oracle.argmax(vals)
        for t in range(3):
            assert got_pos[t] == brute_argmax(vals[t], list(range(n)))


def test_argmax_tie_prefers_lowest_vocab_id_not_position():
    vals = np.array([[1.0, 5.0, 5.0, 2.0]])
    ids = np.array([9, 40, 12, 3], np.int32)
    got, val, gap = oracle.argmax(vals, ids)
    assert got[0] == 12 and val[0] == 5.0 and gap[0] == 0.0


def test_argmax_all_nan_gives_minus_one():
    got, val, _ = oracle.argmax(np.full((2, 3), np.nan))
    assert got.tolist() == [-1, -1] and np.all(np.isnan(val))


def test_argmax_planted_maximum():
    """Row r* is the sign pattern of x at full magnitude; it must win, and a copy
    of it at a higher index must not take the id."""
    N, K = 64, 512
    p, s = synth.weight(29, N, K)
    x = synth.activations(29, 1, K)
    xf = synth.bf16_to_f32(x)[0]
    lev = np.where(xf > 0, 15, 0).astype(np.uint8)
    r_star, r_copy = 17, 41
    p[r_star] = lev[0::2] | (lev[1::2] << 4)
    s[r_star] = bf16_bits(0.5)
    p[r_copy], s[r_copy] = p[r_star], s[r_star]
    y, _ = oracle.matmul(p, s, x)
    got, val, gap = oracle.argmax(y)
    others = np.delete(y[0], [r_star, r_copy])
    assert got[0] == r_star and gap[0] == 0.0 and val[0] > others.max()


def _gap_case(c):
    y = np.array([[float(v) for v in c["y"]]], np.float64)
    ids = None if c["ids"] is None else np.array(c["ids"], np.int32)
    return y, ids, float(c["gap"])


def test_argmax_gap_hand_examples():
    """Non-zero gaps, a best id held at two positions, one id everywhere (+inf),
    NaN and negative scores: the gap is exact, with the right sign, against
    the second id rather than the second position."""
    for c in load("argmax_gap.json")["cases"]:
        y, ids, gap_ref = _gap_case(c)
        got, val, gap = oracle.argmax(y, ids)
        assert got[0] == c["id"] and val[0] == c["val"], c["name"]
        assert gap[0] == gap_ref, (c["name"], gap[0], gap_ref)


def test_argmax_gap_brute_force_tiny():
    """The gap against a brute force over the distinct ids of random rows with
    repeated ids, ties and NaNs."""
    rng = np.random.default_rng(16)
    for _ in range(300):
        n = int(rng.integers(1, 10))
        y = rng.integers(-4, 5, size=(2, n)).astype(np.float64) / 2
        y[rng.random((2, n)) < 0.2] = np.nan
        ids = rng.integers(0, 5, size=n).astype(np.int32)
        got, val, gap = oracle.argmax(y, ids)
        for t in range(2):
            per_id = {}
            for v, i in zip(y[t], ids):
                if not np.isnan(v):
                    per_id[int(i)] = max(per_id.get(int(i), -np.inf), v)
            if not per_id:
                assert got[t] == -1 and np.isnan(gap[t])
                continue
            best = max(per_id.values())
            best_id = min(i for i, v in per_id.items() if v == best)
            others = [v for i, v in per_id.items() if i != best_id]
            assert got[t] == best_id and val[t] == best
            assert gap[t] == (best - max(others) if others else np.inf)


# Plausible slips in the gap, planted in a copy of the oracle's own source
# (the line as written, then the mistake).
GAP_MUTATIONS = {
    "sign_flipped": ("gap_out[t] = have_second ? row[best] - second : INFINITY;",
                     "gap_out[t] = have_second ? second - row[best] : INFINITY;"),
    "second_by_position": ("if (isnan(row[i]) || id == best_id) continue;",
                           "if (isnan(row[i]) || i == best) continue;"),
    "no_other_id_gives_zero": ("gap_out[t] = have_second ? row[best] - second : INFINITY;",
                               "gap_out[t] = have_second ? row[best] - second : 0.0;"),
}


@pytest.mark.parametrize("mutation", sorted(GAP_MUTATIONS))
def test_planted_gap_mistakes_are_caught(tmp_path, mutation):
    """Each planted mistake, compiled from the oracle's source, fails the gap
    pins (and gives the value the fixture says it would)."""
    import ctypes
    import subprocess

    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    before, after = GAP_MUTATIONS[mutation]
    assert src.count(before) == 1, "the line the mutation edits has changed"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(before, after))
    lib_path = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-o", str(lib_path), str(path), "-lm",
                    "-lpthread"], check=True)
    lib = ctypes.CDLL(str(lib_path))
    caught = 0
    for c in load("argmax_gap.json")["cases"]:
        y, ids, gap_ref = _gap_case(c)
        _, _, gap = oracle.argmax(y, ids, lib=lib)
        if gap[0] != gap_ref:
            caught += 1
        if mutation in c.get("wrong", {}):
            assert gap[0] == c["wrong"][mutation], (c["name"], gap[0])
    assert caught > 0, f"the gap pins do not catch {mutation}"


# -------------------------------------------------- planted oracle mistakes ----

def _planted_wrong_order(packed):
    """A plausible slip: high nibble taken as the even column."""
    return ((packed & 0x0F) << 4) | (packed >> 4)


def test_planted_mistakes_are_caught():
    g = load("hand_examples.json")["H1_nibble_order"]
    packed = np.empty((2, 128), np.uint8)
    packed[0], packed[1] = 0x99, 0x0F
    scales = np.array([[bf16_bits(v) for v in r] for r in g["scales"]], np.uint16)
    x = np.empty((2, 256), np.uint16)
    x[0] = bf16_bits(1.0)
    x[1, 0::2], x[1, 1::2] = bf16_bits(1.0), bf16_bits(0.0)
    y_bad, _ = oracle.matmul(_planted_wrong_order(packed), scales, x)
    assert y_bad[1, 1] == g["swapped_order_would_give_y_1_1"] and y_bad.tolist() != g["y"]
    # transposed scale table (groups and rows swapped) breaks the group-boundary example
    h = load("hand_examples.json")["H2_group_boundary"]
    p2 = np.full((2, 128), 0x88, np.uint8)
    p2[0, 63], p2[0, 64] = 0xF8, 0x80
    sc = np.array([[bf16_bits(3.0), bf16_bits(0.5)], [bf16_bits(1.0), bf16_bits(1.0)]], np.uint16)
    y_ok, _ = oracle.matmul(p2, sc, fill_bf16((1, 256), 1.0))
    y_tr, _ = oracle.matmul(p2, np.ascontiguousarray(sc.T), fill_bf16((1, 256), 1.0))
    assert y_ok[0, 0] == h["y"] and y_tr[0, 0] != h["y"]


# ------------------------------------------------------- verify epilogue ----

def _num(v):
    return float("nan") if v == "nan" else (-0.0 if v == "-0" else float(v))


def test_topk_hand_example():
    g = load("verify_epilogue.json")["topk"]
    y = np.array([[_num(v) for v in r] for r in g["scores"]])
    got_id, got_val = oracle.topk(y, g["k"], np.array(g["ids"], np.int32))
    assert got_id.tolist() == g["top_ids"]
    want = np.array([[_num(v) for v in r] for r in g["top_vals"]])
    assert np.array_equal(got_val, want, equal_nan=True)


def test_topk_entry_zero_is_the_argmax():
    rng = np.random.default_rng(11)
    for _ in range(100):
        n = int(rng.integers(1, 40))
        y = rng.integers(-4, 5, size=(3, n)).astype(np.float64)  # many ties
        y[rng.random((3, n)) < 0.2] = np.nan
        ids = rng.permutation(1000)[:n].astype(np.int32)
        top_id, top_val = oracle.topk(y, 5, ids)
        am, av, _ = oracle.argmax(y, ids)
        assert np.array_equal(top_id[:, 0], am)
        assert np.array_equal(top_val[:, 0], av, equal_nan=True)


def test_topk_equals_a_library_sort():
    """numpy's lexsort over (id ascending within score descending) gives the
    same k pairs on random data with ties and NaNs."""
    rng = np.random.default_rng(12)
    for _ in range(50):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, 33))
        y = np.round(rng.normal(size=(2, n)) * 4) / 4
        y[rng.random((2, n)) < 0.1] = np.nan
        ids = rng.permutation(5 * n)[:n].astype(np.int32)
        got_id, got_val = oracle.topk(y, k, ids)
        for t in range(2):
            ok = ~np.isnan(y[t])
            order = np.lexsort((ids[ok], -y[t][ok]))[:k]
            want_id = np.full(k, -1, np.int32)
            want_val = np.full(k, np.nan)
            want_id[:order.size] = ids[ok][order]
            want_val[:order.size] = y[t][ok][order]
            assert np.array_equal(got_id[t], want_id)
            assert np.array_equal(got_val[t], want_val, equal_nan=True)


def test_topk_is_permutation_invariant_and_identity_ids():
    rng = np.random.default_rng(13)
    y = np.round(rng.normal(size=(3, 500)) * 8) / 8
    perm = rng.permutation(500)
    a_id, a_val = oracle.topk(y, 32)
    b_id, b_val = oracle.topk(y[:, perm], 32, perm.astype(np.int32))
    assert np.array_equal(a_id, b_id) and np.array_equal(a_val, b_val)


def test_greedy_hand_examples():
    for case in load("verify_epilogue.json")["greedy"]:
        acc, tok = oracle.greedy_accept(np.array(case["target"], np.int32), np.array(case["draft"], np.int32), 1,
                                        case["rows"])
        assert acc[0] == case["accepted"] and tok[0].tolist() == case["tokens"], case


def test_greedy_accepts_exactly_the_longest_matching_prefix():
    """Properties of the definition on random sequences: every accepted draft
    matches its row's choice, the first unaccepted one does not, and the
    emitted tokens are the choices of rows 0..a."""
    rng = np.random.default_rng(14)
    S, R = 64, 5
    target = rng.integers(0, 4, size=(S, R)).astype(np.int32)
    draft = np.where(rng.random((S, R - 1)) < 0.7, target[:, :R - 1], rng.integers(0, 4, size=(S, R - 1)))
    acc, tok = oracle.greedy_accept(target, draft.astype(np.int32), S, R)
    for s in range(S):
        a = acc[s]
        assert np.array_equal(target[s, :a], draft[s, :a])
        assert a == R - 1 or target[s, a] != draft[s, a]
        assert tok[s, :a + 1].tolist() == target[s, :a + 1].tolist() and np.all(tok[s, a + 1:] == -1)


def test_planted_epilogue_mistakes_are_caught():
    g = load("verify_epilogue.json")
    y = np.array([[_num(v) for v in g["topk"]["scores"][0]]])
    ids = np.array(g["topk"]["ids"], np.int32)
    # ties broken towards the higher id: the fixture's first two ids swap
    keep = ~np.isnan(y[0])
    wrong = np.lexsort((-ids[keep], -y[0][keep]))[:2]
    assert ids[keep][wrong].tolist() == g["topk"]["reversed_tie_order_would_give_row0_first2"]
    assert ids[keep][wrong].tolist() != oracle.topk(y, 2, ids)[0][0].tolist()
    # acceptance that counts every matching draft instead of the matching prefix
    case = g["greedy"][1]
    t, d = np.array(case["target"]), np.array(case["draft"])
    assert int(np.sum(t[:-1] == d)) == 2 and case["accepted"] == 0
    case = g["greedy"][2]
    t, d = np.array(case["target"]), np.array(case["draft"])
    off_by_one = int(np.argmin(np.append(t[:-1] == d, False))) + 1
    assert off_by_one == g["off_by_one_would_give_accepted_for_case_2"] != case["accepted"]


def test_draft_union_hand_example():
    g = load("verify_epilogue.json")["draft_union"]
    ids, m = oracle.draft_union(np.array(g["base"], np.int32), np.array(g["seq"], np.int32), g["n_rows"])
    assert ids.tolist() == g["ids"] and m == g["length"]


def test_draft_union_properties():
    """Set equality with base | valid seq, no repeats among the added ids, base
    kept verbatim, added ids in order of first appearance, -1 padding."""
    rng = np.random.default_rng(15)
    for _ in range(200):
        n_rows = int(rng.integers(1, 60))
        base = rng.permutation(n_rows)[:int(rng.integers(0, n_rows + 1))].astype(np.int32)
        seq = rng.integers(-3, n_rows + 3, size=int(rng.integers(0, 40))).astype(np.int32)
        ids, m = oracle.draft_union(base, seq, n_rows)
        assert ids.size == base.size + seq.size and np.all(ids[m:] == -1)
        assert ids[:base.size].tolist() == base.tolist()
        added = ids[base.size:m]
        valid = [int(v) for v in seq if 0 <= v < n_rows]
        assert set(ids[:m].tolist()) == set(base.tolist()) | set(valid)
        assert len(set(added.tolist())) == added.size and not set(added.tolist()) & set(base.tolist())
        first = [valid.index(int(v)) for v in added]
        assert first == sorted(first)
