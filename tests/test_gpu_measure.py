"""The measurement helper w4a16_stream_read (the streaming-read ceiling that
bench.py prints beside the matmul's weight bandwidth): it must read every
16-byte word of its buffer exactly once.  The XOR of everything it writes to
the sink equals the XOR of all 32-bit words of the buffer exactly when each
word is folded in an odd number of times; with random contents a skipped or
doubled word would change it."""
import numpy as np
import pytest

from gpu_util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_verify_gemv_amd as w4a16
    w4a16.load_library()
    return w4a16


@pytest.mark.parametrize("nbytes,workgroups", [(16, 1), (1 << 20, 7), ((1 << 20) + 48, 13), (3 * 16 * 256 * 4, 2),
                                               (256 << 20, 2048)])
def test_stream_read_reads_every_word_once(w4, nbytes, workgroups):
    say(f"stream_read {nbytes} B over {workgroups} workgroups")
    rng = np.random.default_rng(nbytes + workgroups)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((workgroups * 256,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    w4.stream_read(src, sink, workgroups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_stream_read_rejects_bad_arguments(w4):
    src = torch.zeros(1000, dtype=torch.uint8, device="cuda")  # not a multiple of 16 bytes
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(w4.W4A16Error):
        w4.stream_read(src, sink, 1)
    with pytest.raises(ValueError):
        w4.stream_read(torch.zeros(1024, dtype=torch.uint8, device="cuda"), sink, 2)
