"""Pins of the oracle's asymmetric children and data-free code chooser.

Asymmetric children (MatGPTQ: Efficient and Accurate Inference over Nested
Quantized Models, Tables 4-7 evaluate "asymmetric MatGPTQ"; the pages give no
formula): the reading is that the parent grid is s * (c - z) and a child
value is the mean of its parent bucket.  The pins below check the oracle
against that definition by other routes: the parent grid itself (r = 8), the
bucket mean computed in exact rationals, the reduction to the symmetric
closed form at z = 127.5, and linearity in z.

Code chooser (MatGPTQ: Efficient and Accurate Inference over Nested Quantized
Models, captions of Tables 6 and 7: per-precision weights lambda_3, lambda_4,
lambda_8): the
chosen parent code minimises the lambda-weighted squared error of the
children; ties go to the smallest code.  Pinned by closed forms for a single
width, exact power-of-two scale invariance, sign symmetry and an exact
rational brute force.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def bf16(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def fr_bf16(h):
    return Fraction(float(oracle.bf16_to_f64(np.array([h], dtype=np.uint16))[0]))


# ---------------------------------------------------------------- asymmetric

@pytest.mark.parametrize("r", range(1, 9))
def test_asym_with_midpoint_zero_is_symmetric(r):
    for s in (0.0078125, 0.3, -1.5):
        for q in range(1 << r):
            assert oracle.dequant_value_asym(s, 127.5, q, r) == oracle.dequant_value(s, q, r)


def test_asym_r8_is_parent_grid():
    rng = np.random.default_rng(5)
    for _ in range(200):
        s = float(oracle.bf16_to_f64(bf16([rng.uniform(1e-3, 1.0)]))[0])
        z = float(rng.integers(0, 256))
        c = int(rng.integers(0, 256))
        assert oracle.dequant_value_asym(s, z, c, 8) == s * (c - z)


@pytest.mark.parametrize("r", [1, 2, 3, 4, 6])
def test_asym_child_is_mean_of_parent_bucket(r):
    rng = np.random.default_rng(r)
    for _ in range(20):
        s = fr_bf16(bf16([rng.uniform(1e-3, 1.0)])[0])
        z = fr_bf16(bf16([rng.uniform(-10, 260)])[0])
        q = int(rng.integers(0, 1 << r))
        width = 1 << (8 - r)
        parents = [s * (Fraction(c) - z) for c in range(q * width, (q + 1) * width)]
        mean = sum(parents) / width
        assert Fraction(oracle.dequant_value_asym(float(s), float(z), q, r)) == mean


def _exact_asym(x, codes, scales, zeros, r):
    b, k = x.shape
    n = codes.shape[0]
    xf = [[fr_bf16(v) for v in row] for row in x]
    out = np.empty((b, n), dtype=object)
    width = 1 << (8 - r)
    for i in range(n):
        w = []
        for j in range(k):
            s = fr_bf16(scales[i, j // 128])
            z = fr_bf16(zeros[i, j // 128])
            q = int(codes[i, j]) >> (8 - r)
            # mean of the parent bucket, written out
            w.append(sum(s * (Fraction(c) - z) for c in range(q * width, (q + 1) * width)) / width)
        for bi in range(b):
            out[bi, i] = sum(xf[bi][j] * w[j] for j in range(k))
    return out


@pytest.mark.parametrize("r", [2, 3, 8])
def test_asym_qgemm_exact_rational_bruteforce(r):
    n, k, b = 3, 256, 2
    case = synth.random_case(n, k, b, seed=23)
    rng = np.random.default_rng(23)
    zeros = bf16(rng.integers(0, 256, size=(n, k // 128)).astype(np.float32))
    y = oracle.qgemm_asym(case["x"], oracle.pack(case["codes"]), case["scales"], zeros, n, k, r)
    exact = _exact_asym(case["x"], case["codes"], case["scales"], zeros, r)
    ymax = max(abs(float(v)) for v in exact.reshape(-1))
    assert np.abs(y - exact.astype(np.float64)).max() <= 1e-13 * ymax


def test_asym_qgemm_reduces_to_symmetric_and_is_linear_in_z():
    n, k, b, r = 20, 384, 3, 3
    case = synth.random_case(n, k, b, seed=31)
    planes = oracle.pack(case["codes"])
    half = bf16(np.full((n, k // 128), 127.5, dtype=np.float32))
    sym = oracle.qgemm(case["x"], planes, case["scales"], n, k, r)
    assert np.array_equal(oracle.qgemm_asym(case["x"], planes, case["scales"], half, n, k, r), sym)
    # Y(z1) - Y(z2) = sum_g s_g (z2 - z1) * sum_{k in g} x_k, z1 and z2 integer-valued
    rng = np.random.default_rng(31)
    z1 = rng.integers(0, 256, size=(n, k // 128)).astype(np.float32)
    z2 = rng.integers(0, 256, size=(n, k // 128)).astype(np.float32)
    y1 = oracle.qgemm_asym(case["x"], planes, case["scales"], bf16(z1), n, k, r)
    y2 = oracle.qgemm_asym(case["x"], planes, case["scales"], bf16(z2), n, k, r)
    xs = oracle.bf16_to_f64(case["x"]).reshape(b, k // 128, 128).sum(axis=2)   # [b][G]
    s = oracle.bf16_to_f64(case["scales"])                                     # [n][G]
    expect = xs @ (s * (z2 - z1)).T
    assert np.allclose(y1 - y2, expect, rtol=1e-10, atol=1e-10 * np.abs(expect).max())


def test_asym_rows_select():
    n, k, b, r = 33, 256, 2, 4
    case = synth.random_case(n, k, b, seed=41)
    planes = oracle.pack(case["codes"])
    zeros = bf16(np.random.default_rng(41).integers(100, 150, size=(n, 2)).astype(np.float32))
    full = oracle.qgemm_asym(case["x"], planes, case["scales"], zeros, n, k, r)
    rows = np.array([32, 0, 17])
    assert np.array_equal(oracle.qgemm_asym(case["x"], planes, case["scales"], zeros, n, k, r,
                                            rows=rows), full[:, rows])


# ---------------------------------------------------------------- code chooser

def _scales(n, k, rng, lo=1e-3, hi=1e-2):
    return bf16(rng.uniform(lo, hi, size=(n, k // 128)).astype(np.float32))


def test_choose_single_width8_is_nearest_grid_point():
    rng = np.random.default_rng(7)
    n, k = 6, 256
    s = _scales(n, k, rng)
    sf = oracle.bf16_to_f64(s)
    w = (rng.normal(0, 1, size=(n, k)) * np.repeat(sf, 128, axis=1) * 60).astype(np.float32)
    w[0, :8] = (np.array([-1e3, 1e3, 0, 1, -1, 2, -2, 3]) * sf[0, 0]).astype(np.float32)
    codes = oracle.choose_codes(w, s, [8], [1.0])
    for i in range(n):
        for j in range(k):
            t = Fraction(float(w[i, j])) / Fraction(float(sf[i, j // 128])) + Fraction(255, 2)
            c = int(t) if t >= 0 else int(t) - (0 if t == int(t) else 1)  # floor
            frac = t - c
            if frac > Fraction(1, 2):
                c += 1  # ties (frac == 1/2) keep the smaller code
            c = min(max(c, 0), 255)
            assert codes[i, j] == c, (i, j)


def test_choose_single_width4_takes_first_code_of_nearest_level():
    rng = np.random.default_rng(8)
    n, k = 4, 128
    s = _scales(n, k, rng)
    sf = oracle.bf16_to_f64(s)
    w = (rng.normal(0, 1, size=(n, k)) * np.repeat(sf, 128, axis=1) * 80).astype(np.float32)
    codes = oracle.choose_codes(w, s, [4], [2.5])
    for i in range(n):
        for j in range(k):
            sv = Fraction(float(sf[i, 0]))
            levels = [sv * 16 * (Fraction(q) + Fraction(1, 2) - 8) for q in range(16)]
            err = [abs(Fraction(float(w[i, j])) - L) for L in levels]
            q = err.index(min(err))
            assert codes[i, j] == 16 * q


def test_choose_zero_weight_widths_drop_out():
    rng = np.random.default_rng(9)
    n, k = 3, 256
    s = _scales(n, k, rng)
    w = rng.normal(0, 0.02, size=(n, k)).astype(np.float32)
    a = oracle.choose_codes(w, s, [3, 4, 8], [0.0, 0.0, 1.0])
    b = oracle.choose_codes(w, s, [8], [1.0])
    assert np.array_equal(a, b)


def test_choose_power_of_two_scale_invariance_and_sign_symmetry():
    rng = np.random.default_rng(10)
    n, k = 8, 256
    s = _scales(n, k, rng)
    w = rng.normal(0, 0.02, size=(n, k)).astype(np.float32)
    lam = [0.7, 1.3, 1.0]
    c = oracle.choose_codes(w, s, [3, 4, 8], lam)
    s4 = bf16(oracle.bf16_to_f64(s) * 4)
    assert np.array_equal(oracle.choose_codes(w * 4, s4, [3, 4, 8], lam), c)
    # the grids are symmetric about 0: w -> -w maps code c to 255 - c (random w: no ties)
    assert np.array_equal(oracle.choose_codes(-w, s, [3, 4, 8], lam), 255 - c)


def test_choose_exact_rational_bruteforce():
    rng = np.random.default_rng(11)
    n, k = 2, 128
    s = _scales(n, k, rng)
    w = rng.normal(0, 0.02, size=(n, k)).astype(np.float32)
    widths, lam = [3, 4, 8], [Fraction(4), Fraction(1), Fraction(1, 4)]
    codes = oracle.choose_codes(w, s, widths, [float(v) for v in lam])
    for i in range(n):
        sv = Fraction(float(oracle.bf16_to_f64(s)[i, 0]))
        for j in range(0, k, 7):
            wv = Fraction(float(w[i, j]))
            best, best_loss = None, None
            for c in range(256):
                loss = sum(l * (wv - sv * 2 ** (8 - r) * (Fraction(c >> (8 - r)) + Fraction(1, 2)
                                                            - 2 ** (r - 1))) ** 2
                           for r, l in zip(widths, lam))
                if best is None or loss < best_loss:
                    best, best_loss = c, loss
            assert codes[i, j] == best, (i, j)


def test_choose_rejects_bad_arguments():
    w = np.zeros((2, 128), dtype=np.float32)
    s = np.zeros((2, 1), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.choose_codes(w, s, [3, 4], [1.0])
    with pytest.raises(ValueError):
        oracle.choose_codes(w, s, [9], [1.0])
    with pytest.raises(ValueError):
        oracle.choose_codes(np.zeros((2, 100), dtype=np.float32), s, [8], [1.0])


def test_choose_all_zero_lambdas_tie_to_code_zero():
    rng = np.random.default_rng(12)
    s = _scales(2, 128, rng)
    w = rng.normal(0, 0.02, size=(2, 128)).astype(np.float32)
    assert not oracle.choose_codes(w, s, [3, 4, 8], [0.0, 0.0, 0.0]).any()


@pytest.mark.parametrize("lam", [(1.0, 1.0, 1.0), (4.0, 1.0, 0.25), (0.0, 3.0, 0.5), (9.0, 0.0, 0.0)])
def test_choose_any_nonnegative_lambdas_give_nearest_parent_code(lam):
    # Children are bucket means of the parent grid and buckets are runs of
    # codes, so every child's decision boundaries coincide with the parent
    # grid's: the nearest parent code minimises every term at once (ties and
    # the clamped ends go the same way for every width).
    rng = np.random.default_rng(13)
    n, k = 4, 256
    s = _scales(n, k, rng)
    sf = oracle.bf16_to_f64(s)
    w = (rng.normal(0, 1, size=(n, k)) * np.repeat(sf, 128, axis=1) * 90).astype(np.float32)
    nearest = oracle.choose_codes(w, s, [8], [1.0])
    got = oracle.choose_codes(w, s, [3, 4, 8], list(lam))
    if lam[2] == 0.0:
        # without the 8-bit term only the buckets are fixed: the first code of
        # the nearest code's bucket at the coarsest width with nonzero weight
        rmin = 3 if lam[0] else 4
        nearest = (nearest >> (8 - rmin)) << (8 - rmin)
    assert np.array_equal(got, nearest)
