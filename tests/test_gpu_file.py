"""GPU: a child loaded from the parent file's prefix computes what the in-memory slice does.

The parent is packed on the GPU, written with save_parent, and each child is read
back with load_child (only the file's first file_prefix_bytes(n, k, r) bytes): its
unpacked codes are the parent codes' top r bits (against the oracle), and qgemm on
it is bit-identical to qgemm on slice_view(r) of the packed parent, at batch 1 and 64.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nbw():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nested_bit_weight_amd as m
    m.library()
    return m


@pytest.mark.parametrize("r", [2, 3, 4, 6, 8])
def test_loaded_child_matches_slice(nbw, tmp_path, r):
    n, k = 300, 1024
    case = synth.random_case(n, k, 64, seed=11, recipe="gptq_like", outliers=False)
    codes = torch.from_numpy(case["codes"]).cuda()
    scales = torch.from_numpy(case["scales"]).view(torch.bfloat16).cuda()
    w = nbw.pack_bitplanes(codes)
    path = str(tmp_path / "parent.nbw")
    nbw.save_parent(path, w, scales)
    child, cs = nbw.load_child(path, r)
    assert torch.equal(cs, scales)
    got = nbw.unpack_codes(child, r).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.unpack(oracle.pack(case["codes"]), n, k, r))
    x = torch.from_numpy(case["x"]).view(torch.bfloat16).cuda()
    for b in (1, 64):
        ya = nbw.qgemm(x[:b].contiguous(), child, cs, r)
        yb = nbw.qgemm(x[:b].contiguous(), w.slice_view(r), scales, r)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
