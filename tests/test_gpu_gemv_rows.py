"""The streaming batch-1 kernel at batch 2..4: one launch carries up to four
batch rows in the rows of the matrix-core operand that batch 1 leaves at zero.

Each batch row's sums are formed exactly as in a batch-1 launch (the same
operand row, the same summation order), so a launch over several rows must
match the batch-1 launches of its rows bit for bit; against the fp64 oracle
the design bound of the fp32-accumulation contract applies."""
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
    m.library()  # raises if the HIP library is missing: no fallback
    return m


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((np.abs(y - ref).max(axis=1) / den).max())


def by_rows(nbw, x, child, s, r, **kw):
    """The same product as batch-1 launches, one per batch row."""
    return torch.cat([nbw.qgemm(x[b:b + 1], child, s, r, kernel="gemv", **kw) for b in range(x.shape[0])])


@pytest.mark.parametrize("n,k", [(1000, 1024), (333, 4096), (16, 512), (7, 512)])
@pytest.mark.parametrize("batch", [2, 3, 4, 5, 6, 9])
def test_rows_match_batch1_launches_bitwise(nbw, n, k, batch):
    case = synth.random_case(n, k, batch, seed=100 + batch + k, recipe="gptq_like", outliers=True)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    x = dev(case["x"], torch.bfloat16)
    s = dev(case["scales"], torch.bfloat16)
    planes = oracle.pack(case["codes"])
    for r in (1, 2, 3, 4, 6, 8):
        child = nbw.slice_view(w, r)
        name = nbw.kernel_name(batch, n, k, r, "gemv")
        print(f"gemv rows n={n} k={k} batch={batch} r={r}: {name}", flush=True)
        assert name.startswith("nbw::gemv_kernel<") and ", 4, " in name
        y = nbw.qgemm(x, child, s, r, kernel="gemv")
        y1 = by_rows(nbw, x, child, s, r)
        torch.cuda.synchronize()
        assert torch.equal(y, y1)
        e = rel_err(y.cpu().numpy(), oracle.qgemm(case["x"], planes, case["scales"], n, k, r))
        assert e <= CONTRACT and e <= DESIGN_BOUND, f"r={r} err={e:.3e}"


@pytest.mark.parametrize("batch", [3, 4])
@pytest.mark.parametrize("r", [2, 5, 8])
def test_rows_asymmetric(nbw, batch, r):
    n, k = 250, 2048
    case = synth.random_case(n, k, batch, seed=120 + r)
    rng = np.random.default_rng(121 + r)
    z = synth.f32_to_bf16_bits(rng.integers(96, 160, size=(n, k // 128)).astype(np.float32))
    w = nbw.pack_bitplanes(dev(case["codes"]))
    child = nbw.slice_view(w, r)
    x = dev(case["x"], torch.bfloat16)
    s = dev(case["scales"], torch.bfloat16)
    zd = dev(z, torch.bfloat16)
    y = nbw.qgemm(x, child, s, r, kernel="gemv", zeros=zd)
    y1 = by_rows(nbw, x, child, s, r, zeros=zd)
    torch.cuda.synchronize()
    assert torch.equal(y, y1)
    ref = oracle.qgemm_asym(case["x"], oracle.pack(case["codes"]), case["scales"], z, n, k, r)
    assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("batch", [2, 3, 4])
def test_rows_strided_and_bf16(nbw, out_dtype, batch):
    n, k, r = 136, 1536, 3
    case = synth.random_case(n, k, batch, seed=130 + batch)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    child = nbw.slice_view(w, r)
    s = dev(case["scales"], torch.bfloat16)
    x = dev(case["x"], torch.bfloat16)
    xw = torch.full((batch, k + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    xw[:, 32:32 + k] = x
    xv = xw[:, 32:32 + k]  # row stride k + 64, offset 32 elements (64 bytes)
    yw = torch.full((batch, n + 24), -3.0, dtype=out_dtype, device="cuda")
    yv = yw[:, 8:8 + n]
    nbw.qgemm(xv, child, s, r, out=yv, kernel="gemv", out_dtype=out_dtype)
    dense = nbw.qgemm(x, child, s, r, kernel="gemv", out_dtype=out_dtype)
    rows = by_rows(nbw, x, child, s, r, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(yv, dense) and torch.equal(dense, rows)
    assert bool((yw[:, :8] == -3.0).all()) and bool((yw[:, 8 + n:] == -3.0).all())
    ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, r)
    bound = DESIGN_BOUND if out_dtype == torch.float32 else 2.0 ** -8 + DESIGN_BOUND
    assert rel_err(dense.float().cpu().numpy(), ref) <= bound


@pytest.mark.parametrize("batch", [1, 3, 4])
def test_long_tile_runs_load_x_once_per_set(nbw, batch):
    # 768 tiles over the CUs give each workgroup a run of 3 tiles, and 9 sets
    # over 8 waves two steps per tile: the variant that loads a set's X only
    # with its first tile (the last tile ragged: 11 of 16 rows).  Sampled
    # rows against the oracle, and the batch rows against their batch-1
    # launches bit for bit.
    n, k = 12283, 4608
    rng = np.random.default_rng(140 + batch)
    codes = synth.uniform_codes(n, k, rng)
    x_bits = synth.activations(batch, k, rng)
    scales = synth.uniform_scales(n, k, rng)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n), rng.integers(0, n, 48)]))
    sub_planes = oracle.pack(np.ascontiguousarray(codes[rows]))
    w = nbw.pack_bitplanes(dev(codes))
    x = dev(x_bits, torch.bfloat16)
    s = dev(scales, torch.bfloat16)
    for r in (3, 5):
        child = nbw.slice_view(w, r)
        name = nbw.kernel_name(batch, n, k, r)
        print(f"long runs n={n} k={k} batch={batch} r={r}: {name}", flush=True)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        if 2.5 * cus <= (n + 15) // 16 < 3.5 * cus:  # (runs of 3 tiles on this device)
            assert name.endswith(", true>")
        y = nbw.qgemm(x, child, s, r)
        if batch > 1:
            assert torch.equal(y, by_rows(nbw, x, child, s, r))
        ref = oracle.qgemm(x_bits, sub_planes, np.ascontiguousarray(scales[rows]), len(rows), k, r)
        e = rel_err(y.cpu().numpy()[:, rows], ref)
        assert e <= CONTRACT and e <= DESIGN_BOUND, f"r={r} err={e:.3e}"
