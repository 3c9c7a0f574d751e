"""GPU parity of the full decode weight pass at its real size, in the launch
configuration bench.py times: 64 layers x {qkv, o, gate_up, down} with
distinct seeded weights, repacked to the tiled layout, plus the 248,320-row
lm_head with its per-row argmax, in one grouped launch (the grouped launch's
own tiling for each T).  Outputs are compared with the oracle on sampled rows
of sampled problems (every projection kind, first and last layers, rows at
tile edges); the head's scores in full and its argmax bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_parity, dev, host, sample_rows, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# (layer, projection) pairs whose outputs are checked
CHECKED = [(0, "qkv"), (0, "down"), (17, "gate_up"), (31, "o"), (38, "down"), (63, "gate_up"), (63, "down"),
           (63, "o")]


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    return w4a16


@pytest.fixture(scope="module")
def resident(w4):
    """The bench's resident tiled weights (device only; host copies are
    regenerated from the seeds where a check needs them)."""
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


def check_problems(probs, weights, T, what):
    index = {(layer, proj): i for i, (layer, proj, _) in enumerate(weights)}
    for layer, proj in CHECKED:
        N, K = synth.PROJECTIONS[proj]
        tid = synth.tid_layer(layer, proj)
        p, s = synth.weight(tid, N, K)
        x = synth.activations(tid, T, K)
        rows = sample_rows(N, 48, seed=tid)
        y_ref, a_ref = oracle.gather(rows, p, s, x)
        y = host(probs[index[(layer, proj)]][3])
        r = assert_parity(y[:, rows], y_ref, a_ref, f"{what} layer {layer} {proj}")
        say(f"  layer {layer} {proj}: max err/tol {r:.3g}")


def body_problems(w4, weights, T):
    probs = []
    for layer, proj, tw in weights:
        N, K = synth.PROJECTIONS[proj]
        x = dev(synth.activations(synth.tid_layer(layer, proj), T, K))
        probs.append((tw, None, x, torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")))
    return probs


def test_step_at_t4_with_lm_head_argmax(w4, resident):
    """The bench step: body + lm_head with argmax in one grouped launch."""
    from gpu_util import check_argmax

    weights, head, (hp, hs) = resident
    T = 4
    hn, hk = synth.LM_HEAD
    probs = body_problems(w4, weights, T)
    hx = synth.activations(synth.TID_LM_HEAD, T, hk)
    hy = torch.full((T, hn), float("nan"), dtype=torch.float32, device="cuda")
    hid = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    hval = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
    hws = torch.empty(w4.workspace_bytes(hn, T), dtype=torch.uint8, device="cuda")
    step = w4.Batch(probs + [(head, None, dev(hx), hy, hid, hval, hws)], T)
    say("full pass step T=4 ...")
    step.run()
    torch.cuda.synchronize()
    check_problems(probs, weights, T, "step T=4")
    say("  oracle lm_head T=4 ...")
    y_ref, a_ref = oracle.matmul(hp, hs, hx)
    yh = host(hy)
    r = assert_parity(yh, y_ref, a_ref, "step lm_head T=4")
    say(f"  lm_head: max err/tol {r:.3g}")
    ids = host(hid)
    check_argmax(ids, yh, y_ref, None, "step lm_head T=4")
    assert np.array_equal(host(hval), yh[np.arange(T), ids])
    # the step again: identical bits (no state carried between launches)
    first = [host(y).copy() for *_, y in probs[:8]]
    hid.fill_(-7)
    step.run()
    for f, (*_, y) in zip(first, probs[:8]):
        assert np.array_equal(f, host(y))
    assert np.array_equal(host(hid), ids)


@pytest.mark.parametrize("T", [1, 8, 16])
def test_body_pass_other_widths(w4, resident, T):
    """The body pass alone at the other verify widths bench.py reports."""
    weights, _, _ = resident
    probs = body_problems(w4, weights, T)
    say(f"full pass body T={T} ...")
    w4.Batch(probs, T).run()
    torch.cuda.synchronize()
    check_problems(probs, weights, T, f"body T={T}")
