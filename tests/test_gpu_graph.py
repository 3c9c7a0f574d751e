"""Replays of a captured HIP graph give the eager results, every time.

The library enqueues only kernels (no memset, no allocation, no
synchronisation), so its calls can be captured.  The graph holds single
matmuls in both layouts, grouped launches (one with a problem's argmax),
the gathered head with argmax,
the top-k and greedy acceptance; it is replayed several times with eager
work and synchronisations between the replays, and every replay is compared
bit for bit with the eager run of the same calls.
"""
import numpy as np
import pytest

import synth
from gpu_util import dev, host, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    return w4a16


def test_graph_replays_match_eager(w4):
    T = 4
    p1, s1 = synth.weight(6001, 7168, 5120)
    p2, s2 = synth.weight(6002, 5120, 17408)
    ph, sh = synth.weight(6003, 40000, 5120)
    x1 = dev(synth.activations(6001, T, 5120))
    x2 = dev(synth.activations(6002, T, 17408))
    xh = dev(synth.activations(6003, T, 5120))
    pd1, sd1, pd2, sd2, pdh, sdh = (dev(a) for a in (p1, s1, p2, s2, ph, sh))
    tw1 = w4.repack_tiled(pd1, sd1)
    twh = w4.repack_tiled(pdh, sdh)
    ids = dev(synth.distinct_ids(6004, 9000, 40000))
    y1 = torch.empty((T, 7168), dtype=torch.float32, device="cuda")
    y1t = torch.empty_like(y1)
    y2 = torch.empty((T, 5120), dtype=torch.float32, device="cuda")
    yb1, yb2 = torch.empty_like(y1), torch.empty_like(y2)
    yh = torch.empty((T, 9000), dtype=torch.float32, device="cuda")
    ws = torch.empty(w4.workspace_bytes(9000, T), dtype=torch.uint8, device="cuda")
    tws = torch.empty(w4.topk_workspace_bytes(9000, T, 32), dtype=torch.uint8, device="cuda")
    draft = dev(np.array([1, 2, 3], np.int32))
    batch = w4.Batch([(pd1, sd1, x1, yb1), (pd2, sd2, x2, yb2)], T)
    yba = torch.empty((T, 40000), dtype=torch.float32, device="cuda")
    ba_id = torch.empty(T, dtype=torch.int32, device="cuda")
    ba_val = torch.empty(T, dtype=torch.float32, device="cuda")
    ba_ws = torch.empty(w4.workspace_bytes(40000, T), dtype=torch.uint8, device="cuda")
    yb1t = torch.empty_like(yb1)
    batch_am = w4.Batch([(tw1, None, x1, yb1t), (twh, None, xh, yba, ba_id, ba_val, ba_ws)], T)
    T8 = 12  # a wider grouped launch, mixed layouts
    x8a = dev(synth.activations(6005, T8, 5120))
    x8b = dev(synth.activations(6006, T8, 17408))
    y8a = torch.empty((T8, 7168), dtype=torch.float32, device="cuda")
    y8b = torch.empty((T8, 5120), dtype=torch.float32, device="cuda")
    batch8 = w4.Batch([(tw1, None, x8a, y8a), (pd2, sd2, x8b, y8b)], T8)
    state = {}

    def calls(stream):
        w4.matmul(pd1, sd1, x1, out=y1, stream=stream)
        w4.matmul_tiled(tw1, x1, out=y1t, stream=stream)
        w4.matmul(pd2, sd2, x2, out=y2, stream=stream)
        batch.run(stream)
        batch_am.run(stream)
        batch8.run(stream)
        _, am, av = w4.head_gather_tiled(twh, xh, row_ids=ids, scores=True, argmax=True, out=yh, workspace=ws,
                                         stream=stream)
        ti, tv = w4.topk(yh, 32, row_ids=ids, workspace=tws, stream=stream)
        acc, tok = w4.greedy_accept(am, draft, 1, T, stream=stream)
        state["out"] = (am, av, ti, tv, acc, tok, yb1t, yba, ba_id, ba_val, y8a, y8b)

    def snapshot():
        torch.cuda.synchronize()
        return [host(t).copy() for t in (y1, y1t, y2, yb1, yb2, yh) + state["out"]]

    calls(torch.cuda.current_stream())
    eager = snapshot()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(side)  # warm the plans outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(torch.cuda.current_stream())
    for rep in range(4):
        for t in (y1, y1t, y2, yb1, yb2, yh) + state["out"]:
            t.fill_(-7)  # eager work between replays, and proof the replay rewrote everything
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        say(f"replay {rep}")
        for i, (a, b) in enumerate(zip(got, eager)):
            assert np.array_equal(a, b, equal_nan=True), f"replay {rep}: output {i} differs from the eager run"
