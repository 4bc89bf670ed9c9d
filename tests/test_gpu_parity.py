"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars (from the format definition and the fp32-accumulation contract):
  * pack, slice, unpack: bit-exact;
  * qgemm: for every batch row b, max_n |Y - R| / max_n |R| <= 2e-3 against the
    fp64 oracle R (the contract), and also <= DESIGN_BOUND: the kernels feed
    exact bf16 operands and accumulate in fp32, so only fp32 rounding remains;
  * special cases that fix the rounding: single-group integer problems are
    bit-exact, scaling and sign flips commute bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

CONTRACT = 2e-3
DESIGN_BOUND = 1e-4
KERNELS = ["gemv", "smallb", "gemm"]


@pytest.fixture(scope="module")
def nbw():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nested_bit_weight_amd as m
    m.library()  # raises if the HIP library is missing: no fallback
    print("libnbw", m.version(), flush=True)
    return m


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def rel_err(y, ref):
    """Per batch row: max |y - ref| / max |ref|; returns the max over rows."""
    y = np.asarray(y, dtype=np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((np.abs(y - ref).max(axis=1) / den).max())


def run_qgemm(nbw, case, r, kernel, planes_dev=None):
    n, k = case["n"], case["k"]
    if planes_dev is None:
        w = nbw.pack_bitplanes(dev(case["codes"]))
    else:
        w = planes_dev
    child = nbw.slice_view(w, r)
    x = dev(case["x"], torch.bfloat16)
    s = dev(case["scales"], torch.bfloat16)
    y = nbw.qgemm(x, child, s, r, kernel=kernel)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# ---------------------------------------------------------------- pack / slice

@pytest.mark.parametrize("n,k", [(1, 128), (16, 256), (37, 640), (1000, 1024), (3, 2176)])
def test_pack_bitexact(nbw, n, k):
    codes = synth.uniform_codes(n, k, np.random.default_rng(n * 7 + k))
    w = nbw.pack_bitplanes(dev(codes))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w.storage.cpu().numpy(), oracle.pack(codes))


@pytest.mark.parametrize("r", range(1, 9))
def test_unpack_is_msb_slice(nbw, r):
    n, k = 45, 512
    codes = synth.uniform_codes(n, k, np.random.default_rng(31))
    w = nbw.pack_bitplanes(dev(codes))
    q = nbw.unpack_codes(nbw.slice_view(w, r), r).cpu().numpy()
    np.testing.assert_array_equal(q, codes >> (8 - r))


def test_pack_full_size_tiles(nbw):
    # Llama-3.1-8B gate_up (28672 x 4096): GPU planes vs oracle on tile ranges,
    # plus the full r = 8 round trip on the GPU.
    d = synth.make_linear("llama3.1-8b", 2, 1)
    n, k = d["n"], d["k"]
    w = nbw.pack_bitplanes(dev(d["codes"]))
    np.testing.assert_array_equal(nbw.unpack_codes(w, 8).cpu().numpy(), d["codes"])
    planes = w.storage.cpu().numpy()
    pb = nbw.plane_bytes(n, k)
    tile_bytes = 16 * k // 8
    for t0 in (0, 777, n // 16 - 2):
        ref = oracle.pack(d["codes"][16 * t0:16 * t0 + 32])
        rpb = oracle.plane_bytes(32, k)
        for p in range(8):
            got = planes[p * pb + t0 * tile_bytes:p * pb + (t0 + 2) * tile_bytes]
            np.testing.assert_array_equal(got, ref[p * rpb:(p + 1) * rpb])


# ---------------------------------------------------------------- qgemm parity

SHAPES = [(1000, 1024), (48, 384), (16, 128)]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("r", [1, 2, 3, 4, 5, 6, 7, 8])
def test_qgemm_parity_all_widths(nbw, kernel, r):
    n, k = 1000, 1024
    for b in (1, 2, 5):
        case = synth.random_case(n, k, b, seed=40 + r, recipe="gptq_like", outliers=True)
        y = run_qgemm(nbw, case, r, kernel)
        planes = oracle.pack(case["codes"])
        ref = oracle.qgemm(case["x"], planes, case["scales"], n, k, r)
        e = rel_err(y, ref)
        print(f"kernel={kernel} r={r} b={b} err={e:.3e}", flush=True)
        assert e <= CONTRACT
        assert e <= DESIGN_BOUND


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("batch", [1, 3, 16, 17, 33, 64])
@pytest.mark.parametrize("n,k", SHAPES)
def test_qgemm_parity_batches_and_shapes(nbw, kernel, batch, n, k):
    case = synth.random_case(n, k, batch, seed=50 + batch, recipe="uniform")
    planes = oracle.pack(case["codes"])
    for r in (2, 4, 8):
        y = run_qgemm(nbw, case, r, kernel)
        ref = oracle.qgemm(case["x"], planes, case["scales"], n, k, r)
        e = rel_err(y, ref)
        assert e <= DESIGN_BOUND, f"kernel={kernel} r={r} b={batch} n={n} k={k} err={e:.3e}"


def test_auto_dispatch_large_batch(nbw):
    n, k, b = 300, 512, 256
    case = synth.random_case(n, k, b, seed=61, recipe="gptq_like", outliers=True)
    planes = oracle.pack(case["codes"])
    for r in (3, 8):
        y = run_qgemm(nbw, case, r, "auto")
        ref = oracle.qgemm(case["x"], planes, case["scales"], n, k, r)
        assert rel_err(y, ref) <= DESIGN_BOUND


# ---------------------------------------------------------------- structure

@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("r", [2, 3, 6])
def test_planes_beyond_r_are_not_read(nbw, kernel, r):
    # Poison every plane past the child's r: Y must not change by a single bit.
    n, k, b = 70, 512, 4
    case = synth.random_case(n, k, b, seed=62)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    y0 = run_qgemm(nbw, case, r, kernel, planes_dev=w)
    pb = w.plane_bytes
    for val in (0x00, 0xFF, 0x5A):
        w.storage[r * pb:].fill_(val)
        y1 = run_qgemm(nbw, case, r, kernel, planes_dev=w)
        np.testing.assert_array_equal(y0, y1)
    # the child needs only r planes of storage
    short = torch.empty(r * pb, dtype=torch.uint8, device="cuda")
    short.copy_(w.storage[:r * pb])
    child = nbw.PackedWeight(short, n, k, r)
    y2 = run_qgemm(nbw, case, r, kernel, planes_dev=child)
    np.testing.assert_array_equal(y0, y2)


@pytest.mark.parametrize("kernel", KERNELS)
def test_single_group_integer_case_is_bitexact(nbw, kernel):
    # k = 128, small integer activations and power-of-two scales: every partial
    # sum is an exactly representable fp32 number, so Y must equal the exact
    # result bit for bit (in fp32).
    n, k, b = 32, 128, 4
    rng = np.random.default_rng(63)
    codes = synth.uniform_codes(n, k, rng)
    xi = rng.integers(-8, 9, size=(b, k)).astype(np.float32)
    x = synth.f32_to_bf16_bits(xi)
    s = synth.f32_to_bf16_bits(2.0 ** rng.integers(-8, -3, size=(n, 1)).astype(np.float32))
    case = {"n": n, "k": k, "codes": codes, "x": x, "scales": s}
    planes = oracle.pack(codes)
    for r in (1, 2, 4, 8):
        y = run_qgemm(nbw, case, r, kernel)
        ref = oracle.qgemm(x, planes, s, n, k, r)
        np.testing.assert_array_equal(y, ref.astype(np.float32))


@pytest.mark.parametrize("kernel", KERNELS)
def test_identity_activations_return_weights(nbw, kernel):
    n, k = 40, 256
    case = synth.random_case(n, k, 1, seed=64)
    case["x"] = synth.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    planes = oracle.pack(case["codes"])
    for r in (2, 5, 8):
        y = run_qgemm(nbw, case, r, kernel)
        w = oracle.dequant(planes, case["scales"], n, k, r)
        np.testing.assert_array_equal(y, w.T.astype(np.float32))


@pytest.mark.parametrize("kernel", KERNELS)
def test_metamorphic_scale_and_sign(nbw, kernel):
    n, k, b = 200, 768, 3
    case = synth.random_case(n, k, b, seed=65)
    y = run_qgemm(nbw, case, 4, kernel)
    c2 = dict(case, scales=case["scales"] + np.uint16(1 << 7))     # scales x 2
    np.testing.assert_array_equal(run_qgemm(nbw, c2, 4, kernel), 2 * y)
    cn = dict(case, x=case["x"] ^ np.uint16(0x8000))                # X -> -X
    yn = run_qgemm(nbw, cn, 4, kernel)
    if kernel != "gemm":
        np.testing.assert_array_equal(yn, -y)
    else:
        # The large-batch kernel adds its offset corrections to the running
        # sums on the matrix unit, whose accumulation of products of unlike
        # magnitude is not rounded to nearest and not odd in its inputs
        # (measured on gfx950: negated inputs give a result that is not the
        # negated one in 0.2% to 30% of outputs, by up to an ulp of the
        # running sum).  X -> -X then holds to fp32 rounding only.
        assert rel_err(yn, -y.astype(np.float64)) <= 1e-5
    np.testing.assert_array_equal(run_qgemm(nbw, case, 4, kernel), y)  # run twice


@pytest.mark.parametrize("kernel", KERNELS)
def test_output_canaries_untouched(nbw, kernel):
    n, k, b = 37, 256, 5
    case = synth.random_case(n, k, b, seed=66)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    x = dev(case["x"], torch.bfloat16)
    s = dev(case["scales"], torch.bfloat16)
    guard = 64
    buf = torch.full((b * n + 2 * guard,), 12345.0, dtype=torch.float32, device="cuda")
    y = buf[guard:guard + b * n].view(b, n)
    nbw.qgemm(x, nbw.slice_view(w, 3), s, 3, out=y, kernel=kernel)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:guard] == 12345.0) and np.all(host[-guard:] == 12345.0)
    ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], n, k, 3)
    assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND


def test_zero_batch_is_noop(nbw):
    n, k = 32, 256
    case = synth.random_case(n, k, 1, seed=67)
    w = nbw.pack_bitplanes(dev(case["codes"]))
    x = torch.empty((0, k), dtype=torch.bfloat16, device="cuda")
    s = dev(case["scales"], torch.bfloat16)
    y = nbw.qgemm(x, nbw.slice_view(w, 4), s, 4)
    assert tuple(y.shape) == (0, n)


def test_zero_scale_group(nbw):
    n, k, b = 64, 512, 2
    case = synth.random_case(n, k, b, seed=68)
    case["scales"][:, 2] = 0
    planes = oracle.pack(case["codes"])
    for kernel in KERNELS:
        y = run_qgemm(nbw, case, 5, kernel)
        ref = oracle.qgemm(case["x"], planes, case["scales"], n, k, 5)
        assert rel_err(y, ref) <= DESIGN_BOUND


# ---------------------------------------------------------------- full sizes, sampled

def oracle_rows(d, r, rows):
    """fp64 oracle for the selected output rows only: the oracle packs just those
    rows' codes itself (nothing from the GPU)."""
    sub_codes = np.ascontiguousarray(d["codes"][rows])
    sub_scales = np.ascontiguousarray(d["scales"][rows])
    return oracle.qgemm(d["x"], oracle.pack(sub_codes), sub_scales, len(rows), d["k"], r)


# (every (shape, batch, r) the bench times is checked at full size in
# test_gpu_fullsize.py)


# ---------------------------------------------------------------- grouped launch

def _grouped_case(nbw, specs, seed):
    """specs: list of (n, k, batch, r).  Returns items for qgemm_grouped and host data."""
    items, host = [], []
    for j, (n, k, b, r) in enumerate(specs):
        case = synth.random_case(n, k, b, seed=seed + j, recipe="gptq_like", outliers=b > 2)
        w = nbw.pack_bitplanes(dev(case["codes"]))
        items.append((dev(case["x"], torch.bfloat16), nbw.slice_view(w, r),
                      dev(case["scales"], torch.bfloat16), r))
        host.append((case, r))
    return items, host


def test_grouped_matches_single_launches_and_oracle(nbw):
    # Mixed shapes (ragged n), mixed widths, one grouped dispatch: bit-identical
    # to the single-product kernel (same per-row summation order) and within the
    # design bound of the oracle.
    specs = [(1000, 1024, 1, 4), (48, 384 + 128, 1, 2), (16, 128 * 6, 1, 8), (333, 2048, 1, 3),
             (64, 256, 1, 1), (200, 1024, 1, 6)]
    items, host = _grouped_case(nbw, specs, seed=70)
    outs = nbw.qgemm_grouped(items)
    torch.cuda.synchronize()
    for (x, w, s, r), y, (case, _) in zip(items, outs, host):
        single = nbw.qgemm(x, w, s, r, kernel="gemv")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), single.cpu().numpy())
        ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], case["n"],
                           case["k"], r)
        assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND


def test_grouped_mixed_batches_and_fallbacks(nbw):
    # batch 0 (no-op), batch 3 (the streaming kernel's batch-2..4 launch), odd
    # k/128 (queued on its own)
    specs = [(100, 512, 1, 4), (64, 384, 1, 3), (70, 512, 3, 2), (32, 256, 0, 5), (50, 1024, 1, 2)]
    items, host = _grouped_case(nbw, specs, seed=80)
    outs = nbw.qgemm_grouped(items)
    torch.cuda.synchronize()
    for y, (case, r) in zip(outs, host):
        if case["x"].shape[0] == 0:
            assert tuple(y.shape) == (0, case["n"])
            continue
        ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], case["n"],
                           case["k"], r)
        assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND


def test_grouped_llama8b_layer_sampled(nbw):
    # The four Llama-3.1-8B linears at full size, each with its own width.
    widths = (4, 3, 2, 4)
    items, ds = [], []
    for sid, r in enumerate(widths):
        d = synth.make_linear("llama3.1-8b", sid, 1)
        w = nbw.pack_bitplanes(dev(d["codes"]))
        items.append((dev(d["x"], torch.bfloat16), nbw.slice_view(w, r),
                      dev(d["scales"], torch.bfloat16), r))
        ds.append(d)
    outs = nbw.qgemm_grouped(items)
    torch.cuda.synchronize()
    for (x, w, s, r), y, d in zip(items, outs, ds):
        n = d["n"]
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(n).integers(0, n, 40)]))
        assert rel_err(y.cpu().numpy()[:, rows], oracle_rows(d, r, rows)) <= DESIGN_BOUND


def test_grouped_small_batches_match_single_launches_and_oracle(nbw):
    # Batch 2..16 products with mixed widths (1..8) and ragged n, grouped: the
    # batch-2..4 ones in a dispatch of the streaming kernel, the rest in one of
    # the small-batch kernel.  Each is bit-identical to its single launch (the
    # same kernel and per-output summation order), within the design bound of
    # the oracle.
    specs = [(1000, 1024, 16, 4), (48, 512, 2, 2), (333, 2048, 9, 3), (64, 512, 16, 8),
             (200, 1024, 5, 6), (17, 512, 3, 1), (130, 1536, 12, 5), (96, 512, 7, 7)]
    items, host = _grouped_case(nbw, specs, seed=90)
    outs = nbw.qgemm_grouped(items)
    torch.cuda.synchronize()
    for (x, w, s, r), y, (case, _) in zip(items, outs, host):
        single = nbw.qgemm(x, w, s, r, kernel="gemv" if x.shape[0] <= 4 else "smallb")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), single.cpu().numpy())
        ref = oracle.qgemm(case["x"], oracle.pack(case["codes"]), case["scales"], case["n"],
                           case["k"], r)
        assert rel_err(y.cpu().numpy(), ref) <= DESIGN_BOUND


def test_grouped_llama8b_layer_batch16_mixed_widths_sampled(nbw):
    # The four Llama-3.1-8B linears at full size and batch 16 (the bench's
    # activations), each with its own width, as one grouped dispatch.
    widths = (4, 3, 2, 6)
    wid = synth.WORKLOAD_IDS["llama3.1-8b"]
    items, ds, xs = [], [], []
    for sid, r in enumerate(widths):
        d = synth.make_linear("llama3.1-8b", sid, 1)
        xb = synth.activations(16, d["k"], synth.rng_for(0, wid, sid, synth.T_X))
        w = nbw.pack_bitplanes(dev(d["codes"]))
        items.append((dev(xb, torch.bfloat16), nbw.slice_view(w, r), dev(d["scales"], torch.bfloat16), r))
        ds.append(d)
        xs.append(xb)
    outs = nbw.qgemm_grouped(items)
    torch.cuda.synchronize()
    for (x, w, s, r), y, d, xb in zip(items, outs, ds, xs):
        n = d["n"]
        rows = np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n),
                                         np.random.default_rng(n).integers(0, n, 40)]))
        planes = oracle.pack(np.ascontiguousarray(d["codes"][rows]))
        ref = oracle.qgemm(xb, planes, np.ascontiguousarray(d["scales"][rows]), len(rows), d["k"], r)
        e = rel_err(y.cpu().numpy()[:, rows], ref)
        print(f"grouped b16 {d['name']} r={r} err={e:.3e}", flush=True)
        assert e <= CONTRACT and e <= DESIGN_BOUND
