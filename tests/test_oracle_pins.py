"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every check here is independent of the oracle's own code path: closed forms,
invariants, hand-derived worked examples, exact rational brute force, or a
second route that never touches the bit-planes.  A plausible slip in the oracle
(a wrong plane order, a transposed index, a dropped 1/2, a wrong exponent, a
wrong group index) fails at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _exhaustive_codes(n, k):
    # every code value at every column, and every column class inside a chunk
    i = np.arange(n)[:, None]
    j = np.arange(k)[None, :]
    return ((i * 1 + j * 7 + (j // 128) * 13) % 256).astype(np.uint8)


# ---------------------------------------------------------------- pack / unpack

def test_pack_roundtrip_r8_reconstructs_parent():
    # r = 8 reads all planes and must reproduce the parent codes exactly.
    codes = _exhaustive_codes(259, 256)
    planes = oracle.pack(codes)
    assert planes.size == 8 * oracle.plane_bytes(259, 256)
    np.testing.assert_array_equal(oracle.unpack(planes, 259, 256, 8), codes)


@pytest.mark.parametrize("r", range(1, 9))
def test_child_codes_are_msb_slices(r):
    # MSB slicing: the r-bit child of parent code c is c >> (8 - r), computed here
    # straight from the codes, never from the planes.
    codes = _exhaustive_codes(259, 256)
    planes = oracle.pack(codes)
    np.testing.assert_array_equal(oracle.unpack(planes, 259, 256, r), codes >> (8 - r))


def test_all_256_codes_all_widths_bruteforce():
    # 256 codes x r in 1..8 = 2048 cases, each checked bit for bit.
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    planes = oracle.pack(codes)
    for r in range(1, 9):
        q = oracle.unpack(planes, 2, 128, r)
        for c in range(256):
            assert int(q.reshape(-1)[c]) == c >> (8 - r)


def test_nesting_of_children():
    codes = synth.uniform_codes(40, 384, np.random.default_rng(5))
    planes = oracle.pack(codes)
    for r in range(1, 8):
        np.testing.assert_array_equal(oracle.unpack(planes, 40, 384, r),
                                      oracle.unpack(planes, 40, 384, r + 1) >> 1)


def test_plane_popcounts():
    codes = synth.uniform_codes(45, 512, np.random.default_rng(6))
    planes = oracle.pack(codes)
    pb = oracle.plane_bytes(45, 512)
    for p in range(8):
        plane = planes[p * pb:(p + 1) * pb]
        ones = int(np.unpackbits(plane).sum())
        assert ones == int(((codes >> (7 - p)) & 1).sum())


def test_padding_rows_are_zero_bits():
    # Packing n rows, or the same rows followed by zero codes up to the next
    # multiple of 16, must give the same bytes: padding bits are 0.
    codes = synth.uniform_codes(21, 256, np.random.default_rng(7))
    padded = np.zeros((32, 256), dtype=np.uint8)
    padded[:21] = codes
    np.testing.assert_array_equal(oracle.pack(codes), oracle.pack(padded))


def _golden_layout():
    rows = []
    with open(os.path.join(GOLDEN, "layout_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(tuple(int(v) for v in line.split()))
    return rows


@pytest.mark.parametrize("n,k,p,i,j,byte,bit", _golden_layout())
def test_layout_worked_examples(n, k, p, i, j, byte, bit):
    codes = np.zeros((n, k), dtype=np.uint8)
    codes[i, j] = 1 << (7 - p)
    planes = oracle.pack(codes)
    nz = np.flatnonzero(planes)
    assert nz.tolist() == [byte]
    assert int(planes[byte]) == 1 << bit


# ---------------------------------------------------------------- reads exactly r planes

@pytest.mark.parametrize("r", [1, 2, 3, 4, 6, 8])
def test_child_reads_only_its_prefix(r):
    # "An r-bit model reads exactly r bits": poison every byte past the first r
    # planes; unpack, dequant and qgemm of the r-bit child must not change.
    n, k, b = 35, 256, 3
    case = synth.random_case(n, k, b, seed=11)
    planes = oracle.pack(case["codes"])
    pb = oracle.plane_bytes(n, k)
    ref_q = oracle.unpack(planes, n, k, r)
    ref_w = oracle.dequant(planes, case["scales"], n, k, r)
    ref_y = oracle.qgemm(case["x"], planes, case["scales"], n, k, r)
    for poison in (0x00, 0xFF, None):
        bad = planes.copy()
        if poison is None:
            bad[r * pb:] = np.random.default_rng(3).integers(0, 256, bad.size - r * pb)
        else:
            bad[r * pb:] = poison
        np.testing.assert_array_equal(oracle.unpack(bad, n, k, r), ref_q)
        np.testing.assert_array_equal(oracle.dequant(bad, case["scales"], n, k, r), ref_w)
        np.testing.assert_array_equal(oracle.qgemm(case["x"], bad, case["scales"], n, k, r), ref_y)
        # the child needs only a buffer of r planes
        np.testing.assert_array_equal(oracle.unpack(bad[:r * pb], n, k, r), ref_q)


# ---------------------------------------------------------------- dequant

def test_dequant_r8_is_parent_grid():
    # r = 8: w = s * (c - 127.5), the 8-bit symmetric grid, for every code.
    for s in (1.0, 0.0078125, 0.00341796875):
        for c in range(256):
            assert oracle.dequant_value(s, c, 8) == s * (c - 127.5)


@pytest.mark.parametrize("r", range(1, 9))
def test_child_value_is_mean_of_parent_bucket(r):
    # The r-bit child value is the exact mean of the 2^(8-r) parent values that
    # share its top r bits, hence it lies inside that parent bucket.
    for s in (1.0, 0.005859375):
        width = 1 << (8 - r)
        for q in range(1 << r):
            parents = [Fraction(oracle.dequant_value(s, c, 8)) for c in range(q * width, (q + 1) * width)]
            child = Fraction(oracle.dequant_value(s, q, r))
            assert child == sum(parents) / len(parents)
            assert min(parents) <= child <= max(parents)


@pytest.mark.parametrize("r", range(1, 9))
def test_child_grid_symmetry_and_bound(r):
    s = 0.0068359375
    for q in range(1 << r):
        assert oracle.dequant_value(s, q, r) == -oracle.dequant_value(s, (1 << r) - 1 - q, r)
        for c in range(q << (8 - r), (q + 1) << (8 - r)):
            dev = abs(oracle.dequant_value(s, q, r) - oracle.dequant_value(s, c, 8))
            assert dev <= s * (2 ** (7 - r) - 0.5) + 1e-18


def test_dequant_matrix_matches_values_and_groups():
    # Group g of row i uses scale [i][g]; check against the per-value function
    # with the scale picked by hand for a few entries.
    n, k = 18, 384
    case = synth.random_case(n, k, 1, seed=12)
    planes = oracle.pack(case["codes"])
    w = oracle.dequant(planes, case["scales"], n, k, 4)
    s = oracle.bf16_to_f64(case["scales"])
    for (i, j) in [(0, 0), (0, 127), (0, 128), (17, 383), (9, 256), (16, 200)]:
        q = int(case["codes"][i, j]) >> 4
        assert w[i, j] == oracle.dequant_value(s[i, j // 128], q, 4)


# ---------------------------------------------------------------- qgemm

def _exact_qgemm(x_bits, codes, s_bits, r):
    """Exact rational Y from the codes (MSB slice) and the closed form; tiny inputs only."""
    xf = oracle.bf16_to_f64(x_bits)
    sf = oracle.bf16_to_f64(s_bits)
    b, k = xf.shape
    n = codes.shape[0]
    half = Fraction(1, 2)
    out = np.empty((b, n), dtype=object)
    for bi in range(b):
        for i in range(n):
            acc = Fraction(0)
            for j in range(k):
                q = int(codes[i, j]) >> (8 - r)
                w = Fraction(sf[i, j // 128]) * Fraction(2) ** (8 - r) * (q + half - Fraction(2) ** (r - 1))
                acc += Fraction(xf[bi, j]) * w
            out[bi, i] = acc
    return out


@pytest.mark.parametrize("r", [2, 3, 8])
def test_qgemm_exact_rational_bruteforce(r):
    n, k, b = 5, 256, 3
    case = synth.random_case(n, k, b, seed=13)
    planes = oracle.pack(case["codes"])
    y = oracle.qgemm(case["x"], planes, case["scales"], n, k, r)
    exact = _exact_qgemm(case["x"], case["codes"], case["scales"], r)
    ymax = max(abs(float(v)) for v in exact.reshape(-1))
    for bi in range(b):
        for i in range(n):
            assert abs(y[bi, i] - float(exact[bi, i])) <= 1e-13 * ymax


@pytest.mark.parametrize("r", [1, 4, 6])
def test_qgemm_identity_activations_give_weights(r):
    # X = I (batch = k = 256): Y[b][i] = w[i][b] exactly.
    n, k = 20, 256
    case = synth.random_case(n, k, 1, seed=14)
    planes = oracle.pack(case["codes"])
    eye = synth.f32_to_bf16_bits(np.eye(k, dtype=np.float32))
    y = oracle.qgemm(eye, planes, case["scales"], n, k, r)
    w = oracle.dequant(planes, case["scales"], n, k, r)
    np.testing.assert_array_equal(y, w.T)


@pytest.mark.parametrize("r", [2, 4, 8])
def test_qgemm_second_route_without_planes(r):
    # Route 2: codes -> MSB slice -> fp64 weights -> BLAS product.  It never
    # reads the planes, so a layout or plane-order slip in the oracle shows here.
    n, k, b = 150, 640, 6
    case = synth.random_case(n, k, b, seed=15, recipe="gptq_like", outliers=True)
    planes = oracle.pack(case["codes"])
    y = oracle.qgemm(case["x"], planes, case["scales"], n, k, r)
    q = (case["codes"] >> (8 - r)).astype(np.float64)
    s = np.repeat(oracle.bf16_to_f64(case["scales"]), 128, axis=1)
    w = s * 2.0 ** (8 - r) * (q + 0.5 - 2.0 ** (r - 1))
    y2 = oracle.bf16_to_f64(case["x"]) @ w.T
    assert np.max(np.abs(y - y2)) <= 1e-12 * np.max(np.abs(y2))


def test_qgemm_rows_equals_full():
    n, k, b = 70, 512, 4
    case = synth.random_case(n, k, b, seed=16)
    planes = oracle.pack(case["codes"])
    full = oracle.qgemm(case["x"], planes, case["scales"], n, k, 3)
    rows = [0, 5, 17, 69, 33]
    part = oracle.qgemm_rows(case["x"], planes, case["scales"], n, k, 3, rows)
    np.testing.assert_array_equal(part, full[:, rows])


def test_qgemm_metamorphic_scaling_and_sign():
    n, k, b = 40, 384, 5
    case = synth.random_case(n, k, b, seed=17)
    planes = oracle.pack(case["codes"])
    y = oracle.qgemm(case["x"], planes, case["scales"], n, k, 4)
    # scales x 2 (bf16 exponent + 1) -> Y x 2 exactly
    s2 = case["scales"] + np.uint16(1 << 7)
    np.testing.assert_array_equal(oracle.qgemm(case["x"], planes, s2, n, k, 4), 2 * y)
    # X -> -X (flip the bf16 sign bit) -> Y -> -Y exactly
    xneg = case["x"] ^ np.uint16(0x8000)
    np.testing.assert_array_equal(oracle.qgemm(xneg, planes, case["scales"], n, k, 4), -y)


def test_zero_scale_group_contributes_nothing():
    n, k, b = 16, 256, 2
    case = synth.random_case(n, k, b, seed=18)
    planes = oracle.pack(case["codes"])
    sc = case["scales"].copy()
    sc[:, 1] = 0
    y = oracle.qgemm(case["x"], planes, sc, n, k, 5)
    xs = case["x"].copy()
    xs[:, 128:] = 0
    np.testing.assert_array_equal(y, oracle.qgemm(xs, planes, sc, n, k, 5))


def test_oracle_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((4, 100), dtype=np.uint8))
    with pytest.raises(ValueError):
        oracle.unpack(np.zeros(8 * 512, dtype=np.uint8), 16, 256, 9)
