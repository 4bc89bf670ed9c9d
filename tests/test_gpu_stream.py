"""GPU checks of the two measurement references: the streaming read
(nbw_stream_read) and the matrix-unit rate loop (nbw_mfma_rate).

The read's sink words are per-wave XORs of the 32-bit words each wave read,
so their XOR must equal the XOR of every 32-bit word of the range (numpy on
the host): a read that skipped or repeated a word would change it.  Ragged
sizes cover a range that is not a multiple of one wave's 1 KB row and a range
smaller than one load per wave.

The rate loop's sink holds each thread's sum of its accumulators, so a wave's
64 values add up to iters x the sum of all entries of A_a . B_b over the 64
(a, b) fragment pairs of a round; that sum is sum_k colsum(A)_k rowsum(B)_k,
computed in fp64 from the operand bytes with the instruction's operand layout
(lane l carries k = 8 (l // 32) .. +7 of row / column l % 32).  An instruction
dropped, repeated or fed the wrong fragment changes it.
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


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_mfma_rate_computes_its_products(nbw):
    rng = np.random.default_rng(7)
    vals = rng.standard_normal(16 * 64 * 8).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)          # bf16 by truncation
    ops = torch.from_numpy(bits.view(np.int16)).cuda()
    sink = nbw.mfma_rate_sink()
    sink.fill_(float("nan"))
    iters = 3
    nbw.mfma_rate(ops, iters, sink)
    torch.cuda.synchronize()
    frag = _bf16_to_f64(bits).reshape(16, 64, 8)                    # [fragment][lane][element]
    # sum over the 32 rows (A) or columns (B) for each k = 8 h + e
    ksum = frag.reshape(16, 2, 32, 8).sum(axis=2).reshape(16, 16)   # [fragment][k]
    kabs = np.abs(frag).reshape(16, 2, 32, 8).sum(axis=2).reshape(16, 16)
    want = iters * float(ksum[:8].sum(axis=0) @ ksum[8:].sum(axis=0))
    scale = iters * float(kabs[:8].sum(axis=0) @ kabs[8:].sum(axis=0))
    got = sink.cpu().numpy().astype(np.float64).reshape(-1, 64).sum(axis=1)   # per wave
    assert np.isfinite(got).all()
    assert np.abs(got - want).max() <= 1e-4 * scale, (got[:4], want)
    assert nbw.mfma_rate_flops(sink, iters) == sink.numel() // 64 * iters * 64 * 32768


def test_mfma_rate_rejects_short_buffers(nbw):
    with pytest.raises(ValueError):
        nbw.mfma_rate(torch.zeros(16, dtype=torch.int16, device="cuda"), 1, nbw.mfma_rate_sink())
    with pytest.raises(ValueError):
        nbw.mfma_rate(torch.zeros(8192, dtype=torch.int16, device="cuda"), 1,
                      torch.zeros(16, dtype=torch.float32, device="cuda"))
