"""The parent file format, on the CPU: the r-bit child is a byte prefix of the file.

The pages' sliceable parent loads exactly r bits per weight for an r-bit child
(MatGPTQ: Efficient and Accurate Inference over Nested Quantized Models, Abstract;
Table 1, row "Exact r-bit loading").  The library's file keeps the scales ahead of
the MSB-first planes, so the first file_prefix_bytes(n, k, r) bytes hold the whole
child.  Checked here against the oracle's packing and unpacking (no GPU): the
saved planes are the oracle's planes byte for byte, every child loaded from the
file unpacks to the codes' top r bits, a file cut after the child's prefix still
loads that child (and nothing wider), and damaged headers are refused.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

nbw = pytest.importorskip("nested_bit_weight_amd")


def _parent(n, k, seed):
    rng = np.random.default_rng(seed)
    codes = synth.uniform_codes(n, k, rng)
    planes = oracle.pack(codes)
    scales = synth.f32_to_bf16_bits(rng.uniform(0.001, 0.01, size=(n, k // 128)).astype(np.float32))
    w = nbw.PackedWeight(torch.from_numpy(planes).clone(), n, k, 8)
    s = torch.from_numpy(scales.copy()).view(torch.bfloat16)
    return codes, planes, scales, w, s


def test_prefix_bytes_layout():
    for n, k in [(1, 128), (37, 384), (4096, 14336), (28672, 4096)]:
        pb = (n + 15) // 16 * 16 * k // 8
        planes_at = 4096 + (n * (k // 128) * 2 + 4095) // 4096 * 4096
        for r in range(9):
            assert nbw.file_prefix_bytes(n, k, r) == planes_at + r * pb
    with pytest.raises(ValueError):
        nbw.file_prefix_bytes(16, 100, 4)
    with pytest.raises(ValueError):
        nbw.file_prefix_bytes(16, 128, 9)


@pytest.mark.parametrize("n,k", [(37, 384), (16, 128), (300, 1024)])
def test_round_trip_every_child(tmp_path, n, k):
    codes, planes, scales, w, s = _parent(n, k, seed=n + k)
    path = str(tmp_path / "parent.nbw")
    nbw.save_parent(path, w, s)
    assert os.path.getsize(path) == nbw.file_prefix_bytes(n, k, 8)
    info = nbw.file_info(path)
    assert (info.n, info.k, info.nplanes, info.planes_present) == (n, k, 8, 8)
    pb = int(info.plane_bytes)
    for r in range(1, 9):
        child, cs = nbw.load_child(path, r, device="cpu")
        assert (child.n, child.k, child.nplanes) == (n, k, r)
        got = child.storage.numpy()
        np.testing.assert_array_equal(got, planes[: r * pb])              # the parent's plane prefix
        np.testing.assert_array_equal(oracle.unpack(got, n, k, r), codes >> (8 - r))
        np.testing.assert_array_equal(cs.view(torch.int16).numpy().view(np.uint16), scales)


def test_cut_file_is_a_child_file(tmp_path):
    n, k = 37, 384
    codes, planes, scales, w, s = _parent(n, k, seed=7)
    path = str(tmp_path / "parent.nbw")
    nbw.save_parent(path, w, s)
    data = open(path, "rb").read()
    for r in (2, 3, 6):
        cut = str(tmp_path / f"child{r}.nbw")
        with open(cut, "wb") as f:
            f.write(data[: nbw.file_prefix_bytes(n, k, r)])
        assert nbw.file_info(cut).planes_present == r
        child, _ = nbw.load_child(cut, r, device="cpu")
        np.testing.assert_array_equal(oracle.unpack(child.storage.numpy(), n, k, r), codes >> (8 - r))
        with pytest.raises(ValueError):
            nbw.load_child(cut, r + 1, device="cpu")
    # a cut inside the scales leaves no loadable child
    short = str(tmp_path / "short.nbw")
    with open(short, "wb") as f:
        f.write(data[: 4096 + 10])
    with pytest.raises(nbw.NBWError):
        nbw.file_info(short)


def test_damaged_headers_are_refused(tmp_path):
    n, k = 16, 256
    _, _, _, w, s = _parent(n, k, seed=3)
    path = str(tmp_path / "parent.nbw")
    nbw.save_parent(path, w, s)
    good = bytearray(open(path, "rb").read())

    def refused(mutate, status):
        bad = bytearray(good)
        mutate(bad)
        p = str(tmp_path / "bad.nbw")
        open(p, "wb").write(bytes(bad))
        with pytest.raises(nbw.NBWError) as e:
            nbw.file_info(p)
        assert e.value.status == status

    refused(lambda b: b.__setitem__(0, ord("X")), 1)                      # magic
    refused(lambda b: b.__setitem__(12, 2), 4)                            # layout
    refused(lambda b: b.__setitem__(72, 2), 4)                            # scale type
    refused(lambda b: b.__setitem__(40, b[40] ^ 1), 1)                    # plane bytes
    refused(lambda b: b.__setitem__(64, b[64] ^ 16), 1)                   # planes offset
    refused(lambda b: b.__setitem__(32, 9), 1)                            # planes written
