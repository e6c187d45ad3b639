"""The streaming-read probe (the bench's measured read ceiling) reads every
byte it is given: each workgroup's sink word is the XOR of the 32-bit words
of its contiguous share, recomputed here on the host."""
import numpy as np
import pytest
import torch

from quantized_decode_attention_02_amd import kvq

pytestmark = pytest.mark.gpu


# the last size gives every workgroup more than one pass of 8 x 256 loads
@pytest.mark.parametrize("n_bytes", [16, 4096 * 16 + 48, 3 << 20,
                                     (300 << 20) + 80])
def test_stream_read_xor(n_bytes):
    rng = np.random.default_rng(n_bytes)
    host = rng.integers(0, 1 << 32, size=n_bytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((kvq.STREAM_READ_BLOCKS,), -1, dtype=torch.int32, device="cuda")
    kvq.kvq_stream_read(buf, sink)
    got = sink.cpu().numpy().view(np.uint32)
    n16 = n_bytes // 16
    nb = kvq.STREAM_READ_BLOCKS
    per = -(-n16 // nb)
    # zero words pad the last shares (zero is the XOR identity)
    words = np.zeros(nb * per * 4, dtype=np.uint32)
    words[:n16 * 4] = host[:n16 * 4]
    want = np.bitwise_xor.reduce(words.reshape(nb, per * 4), axis=1)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, bad[:8]
