"""GPU check of the streaming-read reference kernel (uq_stream_read): the XOR of
all 32-bit words it returns equals numpy's, for buffers with a ragged tail, one
pass per block and several passes per block."""
import numpy as np
import pytest

from gpu_util import announce, torch_mod, uq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [4, 4 * 1000 + 12, (1 << 24) + 4 * 7, (1 << 26) + 4])
def test_stream_read_xor(words):
    torch = torch_mod()
    rng = np.random.default_rng(words)
    host = rng.integers(-(1 << 31), 1 << 31, size=words, dtype=np.int64).astype(np.int32)
    announce(f"stream read {words * 4} bytes")
    src = torch.from_numpy(host).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    uq().uq_stream_read(src, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == want
    # XORed into the sink: a second read over the same buffer cancels
    uq().uq_stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
