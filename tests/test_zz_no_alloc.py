"""GPU checks of nbw_qgemm_noalloc, the entry point for callers that cannot
allocate: its split-k partial tiles live in the library's static device
scratch instead of a caller workspace.

Through the C ABI (ctypes), against nbw_qgemm_ex given a caller workspace
(the same kernels and the same fixed split order, so bit-identical Y), on two
calls in a row -- the second with a smaller problem, so it must not depend on
what the first left in the scratch -- and against the fp64 oracle on sampled
rows (max |Y - R| / max |R| per batch row <= 2e-3).  A problem that does not
split (batch 1) passes straight through, and a caller workspace is refused.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

CONTRACT = 2e-3
EINVAL = 1
SCRATCH_BYTES = 64 << 20


@pytest.fixture(scope="module")
def nbw():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nested_bit_weight_amd as m
    m.library()
    return m


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(dtype) if dtype is not None else t).cuda()


def rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((np.abs(y - ref).max(axis=1) / den).max())


def _noalloc(nbw, x, w, s, r, y, opts=None):
    lib = nbw.library()
    o = opts if opts is not None else nbw.QgemmOpts()
    return lib.nbw_qgemm_noalloc(ctypes.c_void_p(x.data_ptr()), x.shape[0], ctypes.byref(w.view),
                                 ctypes.c_void_p(s.data_ptr()), r, ctypes.c_void_p(y.data_ptr()),
                                 ctypes.byref(o),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (batch, n, k, r): the Llama-3.1-8B o shape at batch 256, then a smaller
# problem that also splits k (fewer tiles, fewer groups)
CASES = [(256, 4096, 4096, 4), (128, 1024, 2048, 3)]


def test_noalloc_matches_workspace_path_twice(nbw):
    for i, (batch, n, k, r) in enumerate(CASES):
        need = nbw.workspace_bytes(batch, n, k, r)
        print(f"noalloc case {i}: b={batch} n={n} k={k} r={r} scratch {need} bytes "
              f"({nbw.kernel_name(batch, n, k, r)})", flush=True)
        assert 0 < need <= SCRATCH_BYTES, "the case must split k within the scratch"
        case = synth.random_case(n, k, batch, seed=300 + i, recipe="gptq_like", outliers=True)
        w = nbw.pack_bitplanes(dev(case["codes"]))
        child = nbw.slice_view(w, r)
        x = dev(case["x"], torch.bfloat16)
        s = dev(case["scales"], torch.bfloat16)
        y = torch.full((batch, n), float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc(nbw, x, child, s, r, y) == 0
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
        ref_gpu = nbw.qgemm(x, child, s, r, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, ref_gpu), "scratch and caller workspace must give the same Y"
        rows = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n),
                                         np.random.default_rng(i).integers(0, n, 40)]))
        ref = oracle.qgemm_rows(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, r, rows)
        assert rel_err(y.cpu().numpy()[:, rows], ref) <= CONTRACT


def test_noalloc_without_split_and_refuses_a_workspace(nbw):
    batch, n, k, r = 1, 512, 1024, 4
    case = synth.random_case(n, k, batch, seed=7)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    x = dev(case["x"], torch.bfloat16)
    s = dev(case["scales"], torch.bfloat16)
    y = torch.empty((batch, n), dtype=torch.float32, device="cuda")
    assert _noalloc(nbw, x, nbw.slice_view(w, r), s, r, y) == 0
    ref_gpu = nbw.qgemm(x, nbw.slice_view(w, r), s, r)
    torch.cuda.synchronize()
    assert torch.equal(y, ref_gpu)
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    o = nbw.QgemmOpts(0, 0, 0, 0, None, ws.data_ptr(), ws.numel())
    assert _noalloc(nbw, x, nbw.slice_view(w, r), s, r, y, o) == EINVAL


def test_bench_shapes_fit_the_scratch(nbw):
    for wl in ("llama3.1-8b", "qwen3-8b", "llama-70b"):
        for _, n, k in synth.WORKLOADS[wl]:
            for b in (32, 64, 128, 256):
                for r in (8, 6, 4, 3, 2):
                    assert nbw.workspace_bytes(b, n, k, r) <= SCRATCH_BYTES
