"""GPU parity of the extended products and of the parent-code chooser.

* asymmetric children (zero points) on every kernel against the oracle's
  asymmetric product, within the qgemm contract; with every zero point at
  127.5 they must equal the symmetric kernels bit for bit (the asymmetric
  term is then an exact zero);
* bf16 outputs: |Y - R| <= 2^-8 |R| + 2e-3 max|R| per batch row (the output
  rounding plus the fp32 contract), and the fp32 result of the same kernel
  rounded to nearest even (exactly, where both launches sum in the same
  order);
* strided X and Y (row strides above k and n) give bit-identical results to
  dense operands and leave the gaps between rows untouched;
* the code chooser is bit-exact against the oracle's brute force.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

CONTRACT = 2e-3
KERNELS = ["gemv", "smallb", "gemm"]


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


def zeros_for(n, k, seed, kind="int"):
    rng = np.random.default_rng(seed)
    if kind == "int":
        z = rng.integers(0, 256, size=(n, k // 128)).astype(np.float32)
    else:
        z = rng.uniform(-20.0, 280.0, size=(n, k // 128)).astype(np.float32)
    return synth.f32_to_bf16_bits(z)


# ---------------------------------------------------------------- asymmetric

@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("r", [2, 3, 4, 8])
@pytest.mark.parametrize("batch,n,k", [(1, 200, 1024), (5, 130, 640), (40, 300, 512)])
def test_asym_parity(nbw, kernel, r, batch, n, k):
    case = synth.random_case(n, k, batch, seed=100 + r + batch)
    z = zeros_for(n, k, r + n, "real" if r % 2 else "int")
    print("asym", kernel, r, batch, n, k, flush=True)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    y = nbw.qgemm(dev(case["x"], torch.bfloat16), nbw.slice_view(w, r),
                  dev(case["scales"], torch.bfloat16), r, kernel=kernel,
                  zeros=dev(z, torch.bfloat16))
    torch.cuda.synchronize()
    ref = oracle.qgemm_asym(case["x"], oracle.pack(case["codes"]), case["scales"], z, n, k, r)
    assert rel_err(y.cpu().numpy(), ref) <= CONTRACT
    assert rel_err(y.cpu().numpy(), ref) <= 1e-4  # exact operands, fp32 accumulation


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("r", [3, 8])
def test_asym_midpoint_zero_equals_symmetric_bitwise(nbw, kernel, r):
    n, k, batch = 96, 768, 3 if kernel != "gemv" else 1
    case = synth.random_case(n, k, batch, seed=7 + r)
    half = synth.f32_to_bf16_bits(np.full((n, k // 128), 127.5, dtype=np.float32))
    w = nbw.pack_bitplanes(dev(case["codes"]))
    x = dev(case["x"], torch.bfloat16)
    s = dev(case["scales"], torch.bfloat16)
    ya = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel=kernel, zeros=dev(half, torch.bfloat16))
    ys = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel=kernel)
    torch.cuda.synchronize()
    if kernel != "gemm":
        # the same kernel with the zero-point term switched on: bit-identical
        assert torch.equal(ya, ys)
    else:
        # at large batch symmetric children run on their own kernel (the
        # asymmetric ones on the zero-point variant), so the two sum in
        # different orders: equal up to fp32 rounding, and each within the
        # design bound of the oracle
        ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, r)
        assert rel_err(ya.cpu().numpy(), ys.cpu().numpy().astype(np.float64)) <= 1e-5
        assert rel_err(ya.cpu().numpy(), ref) <= 1e-4 and rel_err(ys.cpu().numpy(), ref) <= 1e-4


# ---------------------------------------------------------------- bf16 output

@pytest.mark.parametrize("kernel,batch", [("gemv", 1), ("smallb", 7), ("smallb", 23), ("gemm", 7), ("gemm", 23)])
@pytest.mark.parametrize("r", [2, 4])
def test_bf16_output(nbw, kernel, batch, r):
    n, k = 250, 1024
    case = synth.random_case(n, k, batch, seed=50 + r)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    x = dev(case["x"], torch.bfloat16)
    s = dev(case["scales"], torch.bfloat16)
    y16 = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel=kernel, out_dtype=torch.bfloat16)
    y32 = nbw.qgemm(x, nbw.slice_view(w, r), s, r, kernel=kernel)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    got = y16.float().cpu().numpy().astype(np.float64)
    f32 = y32.cpu().numpy()
    # exactly the fp32 result rounded to nearest even (both launches take the
    # same path and summation order)
    assert np.array_equal(got, bf16_round(f32))
    ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, r)
    bound = 2.0 ** -8 * np.abs(ref) + CONTRACT * np.abs(ref).max(axis=1, keepdims=True)
    assert np.all(np.abs(got - ref) <= bound)


# ---------------------------------------------------------------- strides

@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_strided_operands_match_dense(nbw, kernel, out_dtype):
    n, k, r = 136, 512, 3
    batch = 1 if kernel == "gemv" else 18
    case = synth.random_case(n, k, batch, seed=77)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    child = nbw.slice_view(w, r)
    s = dev(case["scales"], torch.bfloat16)
    x = dev(case["x"], torch.bfloat16)
    xw = torch.full((batch, k + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    xw[:, 32:32 + k] = x
    xv = xw[:, 32:32 + k]  # row stride k + 64, offset 32 elements (64 bytes)
    yw = torch.full((batch, n + 24), -3.0, dtype=out_dtype, device="cuda")
    yv = yw[:, 8:8 + n]
    nbw.qgemm(xv, child, s, r, out=yv, kernel=kernel, out_dtype=out_dtype)
    dense = nbw.qgemm(x, child, s, r, kernel=kernel, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(yv, dense)
    assert bool((yw[:, :8] == -3.0).all()) and bool((yw[:, 8 + n:] == -3.0).all())


def test_strides_rejected_when_misaligned(nbw):
    n, k = 64, 256
    case = synth.random_case(n, k, 2, seed=1)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    xw = torch.zeros((2, k + 4), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nbw.NBWError):
        nbw.qgemm(xw[:, :k], nbw.slice_view(w, 2), dev(case["scales"], torch.bfloat16), 2)


# ---------------------------------------------------------------- code chooser

def _chooser_case(n, k, seed):
    rng = np.random.default_rng(seed)
    s = synth.f32_to_bf16_bits(rng.uniform(1e-3, 1e-2, size=(n, k // 128)).astype(np.float32))
    sf = oracle.bf16_to_f64(s)
    w = (rng.normal(0, 1, size=(n, k)) * np.repeat(sf, 128, axis=1) * 70).astype(np.float32)
    # edge values: far outside the grid, zero, exact grid points and midpoints
    w[0, :6] = np.array([1e4, -1e4, 0.0, 0.5 * sf[0, 0], -0.5 * sf[0, 0], 1.5 * sf[0, 0]],
                        dtype=np.float32)
    return w, s


@pytest.mark.parametrize("widths,lambdas", [([3, 4, 8], [1.0, 1.0, 1.0]),
                                            ([3, 4, 8], [4.0, 1.0, 0.25]),
                                            ([8], [1.0]),
                                            ([2, 6], [0.3, 0.0]),
                                            ([4, 3], [0.0, 0.0])])
def test_choose_codes_bitexact(nbw, widths, lambdas):
    n, k = 70, 384
    w, s = _chooser_case(n, k, sum(widths))
    got = nbw.choose_codes(dev(w), dev(s, torch.bfloat16), widths, lambdas)
    torch.cuda.synchronize()
    ref = oracle.choose_codes(w, s, widths, lambdas)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_choose_codes_full_shape_sampled(nbw):
    # a Llama-3.1-8B o_proj-sized matrix (4096 x 4096): sampled rows checked
    n, k = 4096, 4096
    w, s = _chooser_case(n, k, 3)
    got = nbw.choose_codes(dev(w), dev(s, torch.bfloat16), [3, 4, 8], [1.0, 1.0, 1.0]).cpu().numpy()
    rows = np.array([0, 1, 777, 2048, 4095])
    ref = oracle.choose_codes(w[rows], s[rows], [3, 4, 8], [1.0, 1.0, 1.0])
    assert np.array_equal(got[rows], ref)
