"""GPU checks of the large-batch GEMM's split-k paths.

When a launch splits k, its splits meet in a caller workspace: each split
stores its partial tile and a second launch adds them in the fixed split
order.  Without a (large enough) workspace the launch runs unsplit.  Checked
here:

* the workspace path against the fp64 oracle (fp32 and bf16 Y, symmetric and
  asymmetric children), within the qgemm contract and the fp32 design bound;
* it is deterministic (two calls bit-identical) and its bf16 Y is exactly its
  fp32 Y rounded to nearest even (same summation order);
* it agrees with the unsplit launch within the design bound, and the unsplit
  launch is deterministic too;
* it needs no initial workspace contents (workspaces start as NaN bytes) and
  a workspace can be reused across calls and shapes;
* a workspace smaller than required leaves it untouched and runs unsplit;
* the plain C entry point nbw_qgemm (no workspace) gives bit-identical Y on
  two calls at a shape whose large-batch launch would split k.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

CONTRACT = 2e-3
DESIGN_BOUND = 1e-4


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


def bf16_round(a):
    return oracle.bf16_to_f64(synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)))


# (batch, n, k): few output tiles and long k, so the launch splits k; in the
# last one 33 groups over 8 requested splits of 5 leave 7 that hold groups
SHAPES = [(256, 512, 4096), (200, 300, 2048), (40, 256, 1536), (128, 256, 4224)]


def nan_workspace(nbytes):
    return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")


def _case(nbw, batch, n, k, seed):
    case = synth.random_case(n, k, batch, seed=seed, recipe="gptq_like", outliers=True)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    return case, w, dev(case["x"], torch.bfloat16), dev(case["scales"], torch.bfloat16)


@pytest.mark.parametrize("batch,n,k", SHAPES)
@pytest.mark.parametrize("r", [8, 4, 2])
def test_workspace_split_matches_oracle(nbw, batch, n, k, r):
    need = nbw.workspace_bytes(batch, n, k, r, "gemm")
    assert need > 0, "the shape must split k"
    case, w, x, s = _case(nbw, batch, n, k, seed=n + r)
    ws = nan_workspace(need)
    y = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel="gemm", workspace=ws)
    y2 = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel="gemm", workspace=ws)
    y16 = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel="gemm", workspace=ws,
                    out_dtype=torch.bfloat16)
    ya = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel="gemm", workspace=None)
    ya2 = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel="gemm", workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(ya, ya2)                                 # unsplit: deterministic too
    ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, r)
    e = rel_err(y.cpu().numpy(), ref)
    print(f"split b={batch} n={n} k={k} r={r} err={e:.3e}", flush=True)
    assert e <= CONTRACT and e <= DESIGN_BOUND
    assert torch.equal(y, y2)                                   # deterministic
    got16 = y16.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got16, bf16_round(y.cpu().numpy()))   # same sum, rounded once
    # (the two launches sum in different orders; each is within the design
    # bound of the oracle, and so is their difference)
    assert rel_err(ya.cpu().numpy(), y.cpu().numpy().astype(np.float64)) <= DESIGN_BOUND


def test_workspace_asymmetric(nbw):
    batch, n, k, r = 256, 512, 4096, 3
    case, w, x, s = _case(nbw, batch, n, k, seed=5)
    z = synth.f32_to_bf16_bits(np.random.default_rng(3).uniform(-20, 280, size=(n, k // 128)).astype(np.float32))
    ws = nan_workspace(nbw.workspace_bytes(batch, n, k, r, "gemm"))
    y = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel="gemm", zeros=dev(z, torch.bfloat16), workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.qgemm_asym(case["x"], oracle.pack(case["codes"]), case["scales"], z, n, k, r)
    assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND


def test_workspace_reused_across_shapes_and_short_workspace_falls_back(nbw):
    need = max(nbw.workspace_bytes(b, n, k, 4, "gemm") for b, n, k in SHAPES)
    ws = nan_workspace(need)
    for rep in range(2):
        for i, (batch, n, k) in enumerate(SHAPES):
            case, w, x, s = _case(nbw, batch, n, k, seed=40 + i)
            y = nbw.qgemm(x, nbw.slice_view(w, 4), s, 4, kernel="gemm", workspace=ws)
            torch.cuda.synchronize()
            ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, 4)
            assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND
    # too small: the launch runs unsplit and is still right
    batch, n, k = SHAPES[0]
    case, w, x, s = _case(nbw, batch, n, k, seed=9)
    small = torch.full((256,), 0x5A, dtype=torch.uint8, device="cuda")
    y = nbw.qgemm(x, nbw.slice_view(w, 4), s, 4, kernel="gemm", workspace=small)
    torch.cuda.synchronize()
    ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, 4)
    assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND
    assert bool((small == 0x5A).all())   # untouched


def test_plain_entry_point_is_deterministic(nbw):
    """nbw_qgemm through the C ABI (no workspace) on the Llama-3.1-8B o shape at
    batch 256, where a launch with a workspace splits k: two calls, bit-identical Y."""
    import ctypes
    batch, n, k, r = 256, 4096, 4096, 4
    assert nbw.workspace_bytes(batch, n, k, r) > 0, "the shape must be one that splits k"
    case, w, x, s = _case(nbw, batch, n, k, seed=77)
    lib = nbw.library()
    view = nbw.slice_view(w, r).view
    ys = []
    for _ in range(2):
        y = torch.full((batch, n), float("nan"), dtype=torch.float32, device="cuda")
        st = lib.nbw_qgemm(ctypes.c_void_p(x.data_ptr()), batch, ctypes.byref(view),
                           ctypes.c_void_p(s.data_ptr()), r, ctypes.c_void_p(y.data_ptr()),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    rows = np.arange(0, n, 61)
    ref = oracle.qgemm_rows(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, r, rows)
    got = ys[0].cpu().numpy()[:, rows].astype(np.float64)
    assert rel_err(got, ref) <= CONTRACT
