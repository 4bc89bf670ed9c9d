"""GPU parity of the small-batch kernel where its step order crosses set boundaries,
and of the automatic choice between it and the large-batch GEMM.

The kernel walks (set, tile) steps set-major and prefetches planes and scales
across set boundaries; a workgroup holds a run of tiles and each wave several
sets.  These shapes make every boundary case meet in one launch:

* n = 6149: 385 tiles, two per workgroup, the last tile ragged (rows past n);
* k = 4224: 33 groups, so k/128 is not a multiple of 4 and the last set holds
  one group (the three groups past k carry scale 0 and repeated activations);
  9 sets over 8 waves, so wave 0 runs two sets;
* batch 7 (rows past the batch in the MFMA tile) and 16, r = 3 and 5 (one and
  two decode phases), plus zero points;
* batch 25 and 32 at r = 3: two 16-row slices per workgroup (32 batch rows per
  pass over the planes), the second one partly past the batch at 25; and with
  zero points at batch 29.

Every output is compared with the fp64 oracle.  Bars as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

CONTRACT = 2e-3
DESIGN_BOUND = 1e-4
N, K = 6149, 4224


@pytest.fixture(scope="module")
def nbw():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nested_bit_weight_amd as m
    m.library()
    return m


@pytest.fixture(scope="module")
def case():
    return synth.random_case(N, K, 32, seed=77, recipe="gptq_like", outliers=True)


def rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((np.abs(y - ref).max(axis=1) / den).max())


@pytest.mark.parametrize("batch,r", [(7, 3), (16, 3), (7, 5), (16, 5), (25, 3), (32, 3)])
def test_smallb_set_boundaries_every_output(nbw, case, batch, r):
    print(f"smallb n={N} k={K} batch={batch} r={r}", flush=True)
    name = nbw.kernel_name(batch, N, K, r)
    print(f"  {name}", flush=True)
    assert name.startswith("nbw::smallb_kernel") and name.endswith(", 2>" if batch > 16 else ", 1>")
    w = nbw.pack_bitplanes(torch.from_numpy(case["codes"]).cuda())
    xb = np.ascontiguousarray(case["x"][:batch])
    x = torch.from_numpy(xb).view(torch.bfloat16).cuda()
    s = torch.from_numpy(case["scales"]).view(torch.bfloat16).cuda()
    y = nbw.qgemm(x, w.slice_view(r), s, r).cpu().numpy()
    assert np.all(np.isfinite(y))
    e = rel_err(y, oracle.qgemm(xb, oracle.pack(case["codes"]), case["scales"], N, K, r))
    print(f"  err={e:.3e}", flush=True)
    assert e <= CONTRACT and e <= DESIGN_BOUND


@pytest.mark.parametrize("batch", [9, 29])
def test_smallb_set_boundaries_asym(nbw, case, batch):
    r = 4
    print(f"smallb asym n={N} k={K} batch={batch} r={r}", flush=True)
    rng = np.random.default_rng(78)
    z = synth.f32_to_bf16_bits(rng.integers(96, 160, size=(N, K // 128)).astype(np.float32))
    w = nbw.pack_bitplanes(torch.from_numpy(case["codes"]).cuda())
    xb = np.ascontiguousarray(case["x"][:batch])
    x = torch.from_numpy(xb).view(torch.bfloat16).cuda()
    s = torch.from_numpy(case["scales"]).view(torch.bfloat16).cuda()
    zd = torch.from_numpy(z).view(torch.bfloat16).cuda()
    y = nbw.qgemm(x, w.slice_view(r), s, r, zeros=zd).cpu().numpy()
    ref = oracle.qgemm_asym(xb, oracle.pack(case["codes"]), case["scales"], z, N, K, r)
    e = rel_err(y, ref)
    print(f"  err={e:.3e}", flush=True)
    assert e <= CONTRACT and e <= DESIGN_BOUND


# The automatic choice: the streaming kernel up to batch 4; the small-batch
# kernel while it needs one pass over the planes (32 batch rows a pass for
# r <= 4 on short tile runs, 16 otherwise), or two passes with k <= 8192; the
# large-batch GEMM beyond.
@pytest.mark.parametrize("batch,k,r,family", [
    (2, 1024, 3, "gemv"), (4, 1024, 6, "gemv"), (4, 8320, 2, "gemv"), (5, 1024, 3, "smallb"),
    (5, 8320, 6, "smallb"),
    (17, 1024, 3, "smallb"), (32, 1024, 3, "smallb"), (33, 1024, 3, "smallb"), (64, 1024, 3, "smallb"),
    (65, 1024, 3, "gemm"), (32, 8320, 3, "smallb"), (33, 8320, 3, "gemm"),
    (17, 1024, 6, "smallb"), (32, 1024, 6, "smallb"), (33, 1024, 6, "gemm"), (17, 8320, 6, "gemm")])
def test_auto_dispatch_boundaries(nbw, batch, k, r, family):
    n = 300
    name = nbw.kernel_name(batch, n, k, r)
    print(f"auto n={n} k={k} batch={batch} r={r}: {name}", flush=True)
    # (the large-batch family: gemm_kernel for asymmetric children,
    # gemm_wide_kernel for symmetric ones)
    assert name.startswith(f"nbw::{family}_") and "_kernel<" in name
    c = synth.random_case(n, k, batch, seed=80 + batch, recipe="gptq_like", outliers=True)
    w = nbw.pack_bitplanes(torch.from_numpy(c["codes"]).cuda())
    x = torch.from_numpy(c["x"]).view(torch.bfloat16).cuda()
    s = torch.from_numpy(c["scales"]).view(torch.bfloat16).cuda()
    y = nbw.qgemm(x, w.slice_view(r), s, r).cpu().numpy()
    e = rel_err(y, oracle.qgemm(c["x"], oracle.pack(c["codes"]), c["scales"], n, k, r))
    print(f"  err={e:.3e}", flush=True)
    assert e <= CONTRACT and e <= DESIGN_BOUND
