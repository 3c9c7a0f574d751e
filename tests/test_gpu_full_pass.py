"""GPU parity of the full decode weight pass at its real size, in the launch
configuration bench.py times: 64 layers x {qkv, o, gate_up, down} with
distinct seeded weights, repacked to the tiled layout, plus the 248,320-row
lm_head with its per-row argmax, in one grouped launch (the grouped launch's
own tiling for each T).  Every one of the 256 body problems is compared with
the oracle on its first and last 16-row tiles and a few random rows; the
head's scores in full and its argmax bit for bit.  Outputs start as NaN, so
an unwritten row fails.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, check_argmax, dev, host, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    return w4a16


@pytest.fixture(scope="module")
def resident(w4):
    """The bench's resident tiled weights (device only; the rows a check
    needs are regenerated on the host from the seeds)."""
    say("full pass: 64 layers + lm_head to the device ...")
    weights = []
    for layer in range(synth.LAYERS):
        for proj in synth.PROJ_ORDER:
            N, K = synth.PROJECTIONS[proj]
            p, s = synth.weight(synth.tid_layer(layer, proj), N, K)
            weights.append((layer, proj, w4.repack_tiled(dev(p), dev(s))))
            del p, s
    hn, hk = synth.LM_HEAD
    hp, hs = synth.weight(synth.TID_LM_HEAD, hn, hk)
    head = w4.repack_tiled(dev(hp), dev(hs))
    torch.cuda.synchronize()
    yield weights, head, (hp, hs)
    del weights, head
    torch.cuda.empty_cache()


def checked_rows(N: int, seed: int, extra: int = 6) -> np.ndarray:
    """The first and last 16-row tiles and `extra` random rows of an N-row matrix."""
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(16), np.arange(N - 16, N), rng.choice(np.arange(16, N - 16), extra, False)])
    return np.unique(rows).astype(np.int64)


def check_all_problems(probs, weights, T, what):
    """Every body problem against the oracle on its checked rows."""
    worst = 0.0
    for (layer, proj, _), prob in zip(weights, probs):
        N, K = synth.PROJECTIONS[proj]
        tid = synth.tid_layer(layer, proj)
        rows = checked_rows(N, seed=tid * 31 + T)
        p, s = synth.weight_rows(tid, rows, K)
        x = synth.activations(tid, T, K)
        y_ref, a_ref = oracle.matmul(p, s, x)
        y = host(prob[3])
        worst = max(worst, assert_parity(y[:, rows], y_ref, a_ref, f"{what} layer {layer} {proj}"))
    say(f"  {what}: all {len(probs)} body problems checked, max err/tol {worst:.3g}")


def body_problems(w4, weights, T):
    probs = []
    for layer, proj, tw in weights:
        N, K = synth.PROJECTIONS[proj]
        x = dev(synth.activations(synth.tid_layer(layer, proj), T, K))
        probs.append((tw, None, x, torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")))
    return probs


@pytest.mark.parametrize("T", [1, 4, 8])
def test_step_with_lm_head_argmax(w4, resident, T):
    """The bench step at T = 1, 4 and 8: body + lm_head with argmax in one
    grouped launch; all 257 problems checked."""
    weights, head, (hp, hs) = resident
    hn, hk = synth.LM_HEAD
    probs = body_problems(w4, weights, T)
    hx = synth.activations(synth.TID_LM_HEAD, T, hk)
    hy = torch.full((T, hn), float("nan"), dtype=torch.float32, device="cuda")
    hid = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    hval = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
    hws = torch.empty(w4.workspace_bytes(hn, T), dtype=torch.uint8, device="cuda")
    step = w4.Batch(probs + [(head, None, dev(hx), hy, hid, hval, hws)], T)
    say(f"full pass step T={T} ...")
    step.run()
    torch.cuda.synchronize()
    check_all_problems(probs, weights, T, f"step T={T}")
    say(f"  oracle lm_head T={T} ...")
    y_ref, a_ref = oracle.matmul(hp, hs, hx)
    yh = host(hy)
    r = assert_parity(yh, y_ref, a_ref, f"step lm_head T={T}")
    say(f"  lm_head: max err/tol {r:.3g}")
    ids = host(hid)
    check_argmax(ids, yh, y_ref, None, f"step lm_head T={T}")
    assert np.array_equal(host(hval), yh[np.arange(T), ids])
    # the step again: identical bits (no state carried between launches)
    first = [host(y).copy() for *_, y in probs[:8]]
    hid.fill_(-7)
    step.run()
    for f, (*_, y) in zip(first, probs[:8]):
        assert np.array_equal(f, host(y))
    assert np.array_equal(host(hid), ids)


def test_body_pass_t16(w4, resident):
    """The body pass alone at T = 16 (the widest verify block), every problem checked."""
    weights, _, _ = resident
    T = 16
    probs = body_problems(w4, weights, T)
    say(f"full pass body T={T} ...")
    w4.Batch(probs, T).run()
    torch.cuda.synchronize()
    check_all_problems(probs, weights, T, f"body T={T}")
