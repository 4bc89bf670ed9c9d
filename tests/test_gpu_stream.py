"""GPU check of the streaming-read bandwidth reference (nbw_stream_read).

The sink words are per-wave XORs of the 32-bit words each wave read, so their
XOR must equal the XOR of every 32-bit word of the range (numpy on the host):
a read that skipped or repeated a word would change it.  Ragged sizes cover a
range that is not a multiple of one wave's 1 KB row and a range smaller than
one load per wave.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nbw():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nested_bit_weight_amd as m
    m.library()
    return m


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, 1 << 20, 29 * (1 << 20) + 1024 * 13 + 16])
def test_stream_read_covers_every_word_once(nbw, nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=max(nbytes // 4, 4) + 64, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = nbw.stream_sink()
    sink.fill_(-1)
    nbw.stream_read(src, nbytes, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host[: nbytes // 4]) if nbytes else np.uint32(0)
    assert int(got) == int(want)


def test_stream_read_rejects_short_sink(nbw):
    src = torch.zeros(1024, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        nbw.stream_read(src, 4096, torch.zeros(16, dtype=torch.int32, device="cuda"))
