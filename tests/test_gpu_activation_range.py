"""GPU parity for activations anywhere in the finite bf16 range.

The library keeps the activations in bf16 and multiplies them with exact
bf16 levels, so every product (q - 8) * x is exact in fp32 whatever the
spread of magnitudes inside a row.  Each case plants values into seeded
N(0,1) activation rows:

  * a huge value (2^40, 2^80, 2^126, the largest finite bf16, either sign) at
    columns where every weight row has code 8, so it contributes nothing and
    the exact result is the N(0,1) rest -- a kernel that scaled or rounded a
    row to fit its largest value would lose the rest;
  * bf16 subnormals and values near 2^-120 on non-zero weights (their
    products are far below the 1e-6 absolute term of the tolerance);
  * a large value (2^60) on non-zero weights (large but finite results).

Every path runs: single launches with both kernel variants (the dot variant
up to T = 8), the tiled layout, the gathered head with argmax, and grouped
launches of both layouts, at T from 1 to 16 and K from one group to several
staged slices.  Expected values come only from the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, check_argmax, dev, host, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_MAX = 0x7F7F  # largest finite bf16, 3.3895e38
HUGE = [2.0 ** 40, -(2.0 ** 80), 2.0 ** 126, None]  # None: the largest finite bf16, negated


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    yield w4a16
    w4a16.set_variant("auto")


def planted_case(tid: int, N: int, K: int, T: int):
    """Weights with code 8 in every row at the outlier columns, and
    activations with huge values there (and tiny / large ones elsewhere)."""
    p, s = synth.weight(tid, N, K)
    x = synth.activations(tid, T, K).copy()
    rng = np.random.default_rng(tid)
    outl = np.unique(np.concatenate([[0, K - 1], rng.choice(K, size=min(6, K), replace=False)]))
    for k in outl:
        if k % 2 == 0:
            p[:, k // 2] = (p[:, k // 2] & 0xF0) | 0x08
        else:
            p[:, k // 2] = (p[:, k // 2] & 0x0F) | 0x80
    for t in range(T):
        for j, k in enumerate(outl):
            v = HUGE[(t + j) % len(HUGE)]
            x[t, k] = (BF16_MAX | 0x8000) if v is None else synth.bf16_from_double(v)
    free = np.setdiff1d(np.arange(K), outl)
    for t in range(T):
        if t % 3 == 1:  # subnormal bf16 and values near 2^-120 on ordinary weights
            cols = rng.choice(free, size=min(40, free.size), replace=False)
            x[t, cols[:20]] = rng.integers(1, 0x80, size=cols[:20].size, dtype=np.uint16) | (
                rng.integers(0, 2, size=cols[:20].size, dtype=np.uint16) << 15)
            x[t, cols[20:]] = [synth.bf16_from_double(v) for v in rng.normal(size=cols[20:].size) * 2.0 ** -120]
        if t % 3 == 2 and free.size > 4:  # a large value on ordinary weights
            x[t, free[free.size // 2]] = synth.bf16_from_double(2.0 ** 60)
    return p, s, x


SHAPES = [(64, 128, 1), (300, 1024, 3), (200, 5120, 8), (96, 17408, 8), (130, 2304, 5), (64, 17408, 16),
          (50, 1152, 12), (1100, 5120, 4)]


@pytest.mark.parametrize("N,K,T", SHAPES)
def test_single_launches_both_variants_and_layouts(w4, N, K, T):
    tid = 7000 + N + K + T
    p, s, x = planted_case(tid, N, K, T)
    y_ref, a_ref = oracle.matmul(p, s, x)
    assert np.all(np.isfinite(y_ref))
    pd, sd, xd = dev(p), dev(s), dev(x)
    for variant in ("mfma", "dot"):
        w4.set_variant(variant)
        say(f"range N={N} K={K} T={T} {variant}")
        r = assert_parity(host(w4.matmul(pd, sd, xd)), y_ref, a_ref, f"{variant} N={N} K={K} T={T}")
        say(f"  max err/tol {r:.3g}")
    w4.set_variant("auto")
    tw = w4.repack_tiled(pd, sd)
    r = assert_parity(host(w4.matmul_tiled(tw, xd)), y_ref, a_ref, f"tiled N={N} K={K} T={T}")
    say(f"  tiled max err/tol {r:.3g}")


@pytest.mark.parametrize("T", [1, 4, 16])
def test_gathered_head_with_argmax(w4, T):
    N, K = 6000, 5120
    tid = 7100 + T
    p, s, x = planted_case(tid, N, K, T)
    ids = synth.distinct_ids(tid, 2500, N)
    y_ref, a_ref = oracle.gather(ids, p, s, x)
    pd, sd, xd = dev(p), dev(s), dev(x)
    for variant in ("mfma", "dot"):
        w4.set_variant(variant)
        say(f"range head T={T} {variant}")
        y, am, _ = w4.head_gather(pd, sd, xd, row_ids=dev(ids), argmax=True)
        y, am = host(y), host(am)
        assert_parity(y, y_ref, a_ref, f"head {variant} T={T}")
        check_argmax(am, y, y_ref, ids, f"range head {variant} T={T}")
    w4.set_variant("auto")
    tw = w4.repack_tiled(pd, sd)
    y, am, _ = w4.head_gather_tiled(tw, xd, row_ids=dev(ids), argmax=True)
    y, am = host(y), host(am)
    assert_parity(y, y_ref, a_ref, f"tiled head T={T}")
    check_argmax(am, y, y_ref, ids, f"range tiled head T={T}")


@pytest.mark.parametrize("T", [1, 4, 8, 9, 16])
@pytest.mark.parametrize("tiled", [False, True])
def test_grouped_launch(w4, T, tiled):
    """Problems of several K in one grouped launch (T = 9 and 16: where the
    grouped launch once staged pre-converted activations)."""
    shapes = [(256, 5120), (160, 17408), (48, 1024), (1040, 5120)]
    probs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        tid = 7200 + 10 * i + T
        p, s, x = planted_case(tid, N, K, T)
        refs.append(oracle.matmul(p, s, x))
        pd, sd = dev(p), dev(s)
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        probs.append((w4.repack_tiled(pd, sd), None, dev(x), y) if tiled else (pd, sd, dev(x), y))
    say(f"range grouped T={T} tiled={tiled}")
    batch = w4.Batch(probs, T)
    batch.run()
    for (N, K), prob, (y_ref, a_ref) in zip(shapes, probs, refs):
        assert_parity(host(prob[3]), y_ref, a_ref, f"grouped T={T} tiled={tiled} {N}x{K}")
