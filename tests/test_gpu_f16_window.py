"""GPU parity at the edges of the fp16 level form's window.

Workgroups that stage activations convert them to fp16 times a power of two
2^E when that is exact for every value of the staged slice (8 significant
bits survive from 2^-17 to 65280 after scaling): first with E = 4, and when
a value misses that window, with the E that the slice's largest and
smallest nonzero magnitudes allow; otherwise the slice runs with bf16
levels.  Each case here builds activations whose slices span a controlled
range, repeated in every 128-column group so that every slice of every
tiling sees it:

  * bulk values of magnitude in [2^B, 2^(B+1)) (B = 16), and in each group
    one value 1.9921875 * 2^(B+16) (all mantissa bits set) and one value
    1.9921875 * 2^(B-16): a span of 32 binades that exactly one E fits; with
    the small one a binade lower (B-17) no E fits and the bf16 levels run;
  * two weight rows isolate the two values: every code is 8 except at their
    columns (level 7, scale 0.5).  If E were one too large, the largest value
    would overflow fp16 (about 50% error in its row); one too small, the
    smallest would lose its last bit (0.4% error in its row, against the
    tolerance's 0.1%);
  * a bulk at 2^-60 (E = 59), and one at 2^100 whose span needs E = -101,
    outside |E| <= 100 (bf16 levels).

Single launches of every workgroup shape the planner picks (split waves
with and without the register prefetch, shared workgroups, runs of tiles,
sliced K), both layouts, T from 1 to 16, and grouped launches.  Expected
values come only from the oracle.
"""
import numpy as np
import pytest

import oracle
from gpu_util import assert_parity, dev, host, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOP = 0x7F  # all seven stored mantissa bits


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    w4a16.set_variant("mfma")
    yield w4a16
    w4a16.set_variant("auto")


def bf16_bits(exp2: int, mant: int, neg: bool = False) -> int:
    """bf16 bits of (1 + mant/128) * 2^exp2 (a normal number)."""
    assert -126 <= exp2 <= 127 and 0 <= mant < 128
    return (0x8000 if neg else 0) | ((127 + exp2) << 7) | mant


def window_case(seed: int, N: int, K: int, T: int, bulk: int, lo: int, hi: int):
    """Codes, scales and activations: bulk magnitudes [2^bulk, 2^(bulk+1)),
    in every group one value at 2^hi and one at 2^lo (mantissa bits all set);
    weight row 0 sees only the 2^lo values, row 1 only the 2^hi values."""
    rng = np.random.default_rng(seed)
    G = K // 128
    packed = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = np.full((N, G), 0x3C80, dtype=np.uint16)  # 0.015625
    scales[:, ::3] = 0x3D4D                              # 0.05, mixed in
    x = np.empty((T, K), dtype=np.uint16)
    mant = rng.integers(0, 128, size=(T, K), dtype=np.uint16)
    sign = rng.integers(0, 2, size=(T, K), dtype=np.uint16) << 15
    x[:] = sign | np.uint16((127 + bulk) << 7) | mant
    t_lo, t_hi = 0, T - 1
    c_lo = np.arange(G) * 128 + 5
    c_hi = np.arange(G) * 128 + 77
    x[t_lo, c_lo] = bf16_bits(lo, TOP)
    x[t_hi, c_hi] = bf16_bits(hi, TOP, neg=True)

    def isolate(row, cols):
        codes = np.full(K, 8, dtype=np.uint8)
        codes[cols] = 15  # level 7
        packed[row] = codes[0::2] | (codes[1::2] << 4)
        scales[row] = 0x3F00  # 0.5

    isolate(0, c_lo)
    isolate(1, c_hi)
    return packed, scales, x


CASES = [  # (bulk, lo, hi): one E fits / none fits / far from 1 / out of |E| <= 100
    ("fits", 16, 0, 32),
    ("no_fit", 16, -1, 32),
    ("tiny", -60, -76, -44),
    ("huge", 100, 84, 116),
]
SHAPES = [(300, 5120, 1), (300, 5120, 2), (96, 17408, 2), (300, 5120, 4), (1100, 5120, 3), (300, 17408, 8),
          (1100, 5120, 8), (4200, 5120, 4), (4200, 5120, 8), (160, 17408, 16), (1100, 5120, 16)]


@pytest.mark.parametrize("name,bulk,lo,hi", CASES)
@pytest.mark.parametrize("N,K,T", SHAPES)
def test_single_launches_at_window_edges(w4, name, bulk, lo, hi, N, K, T):
    seed = 8000 + N + K + T + bulk
    p, s, x = window_case(seed, N, K, T, bulk, lo, hi)
    y_ref, a_ref = oracle.matmul(p, s, x)
    assert np.all(np.isfinite(y_ref))
    if name in ("fits", "no_fit"):
        # the isolating rows' results are far above the absolute tolerance,
        # so a lost last bit or an overflow there fails
        assert abs(y_ref[0, 0]) > 100 and abs(y_ref[T - 1, 1]) > 1e9
    pd, sd, xd = dev(p), dev(s), dev(x)
    say(f"window {name} N={N} K={K} T={T}")
    assert_parity(host(w4.matmul(pd, sd, xd)), y_ref, a_ref, f"{name} row-major N={N} K={K} T={T}")
    tw = w4.repack_tiled(pd, sd)
    assert_parity(host(w4.matmul_tiled(tw, xd)), y_ref, a_ref, f"{name} tiled N={N} K={K} T={T}")


@pytest.mark.parametrize("name,bulk,lo,hi", CASES[:2])
@pytest.mark.parametrize("T", [1, 2, 4, 8, 16])
def test_grouped_launch_at_window_edges(w4, name, bulk, lo, hi, T):
    """A grouped launch of tiled problems: shared workgroups up to T = 2, runs
    of tiles above, the 17,408-column problem in sliced shared workgroups."""
    shapes = [(300, 5120), (160, 17408), (1100, 5120)]
    probs, refs = [], []
    for i, (N, K) in enumerate(shapes):
        p, s, x = window_case(8100 + 10 * i + T, N, K, T, bulk, lo, hi)
        refs.append(oracle.matmul(p, s, x))
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
        probs.append((w4.repack_tiled(dev(p), dev(s)), None, dev(x), y))
    say(f"window grouped {name} T={T}")
    w4.Batch(probs, T).run()
    for (N, K), prob, (y_ref, a_ref) in zip(shapes, probs, refs):
        assert_parity(host(prob[3]), y_ref, a_ref, f"grouped {name} T={T} {N}x{K}")


@pytest.mark.parametrize("tile", ["split,1,2", "split,2,8", "shared,1,4", "shared,4,4", "run,3,4"])
@pytest.mark.parametrize("T", [1, 2, 5, 16])
def test_forced_tiles_at_window_edges(w4, tile, T):
    """Tilings the planner leaves alone at these shapes: split waves staging
    more than their register prefetch holds (two waves over 68 groups at
    K = 17,408), two-tile split workgroups, shared workgroups of one and of
    four tiles per wave, runs."""
    try:
        w4.set_tile(tile)
        for name, bulk, lo, hi in CASES[:2]:
            for N, K in [(700, 17408), (700, 5120)]:
                p, s, x = window_case(8200 + N + K + T, N, K, T, bulk, lo, hi)
                y_ref, a_ref = oracle.matmul(p, s, x)
                pd, sd, xd = dev(p), dev(s), dev(x)
                say(f"window tile={tile} {name} N={N} K={K} T={T}")
                assert_parity(host(w4.matmul(pd, sd, xd)), y_ref, a_ref, f"{tile} {name} row-major {N}x{K} T={T}")
                tw = w4.repack_tiled(pd, sd)
                assert_parity(host(w4.matmul_tiled(tw, xd)), y_ref, a_ref, f"{tile} {name} tiled {N}x{K} T={T}")
    finally:
        w4.set_tile(None)
