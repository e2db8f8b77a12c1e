"""Pins of the oracle's Lloyd-Max codebooks and gain-shape quantizer: the
closed-form 1-bit quantizer, J. Max's 1960 table, the optimality conditions
checked by numerical integration, the Panter-Dite high-rate constant, and the
float32 decision rule."""
import math
import os

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

from oracle import codebook_f32, dequantize, gains_f32, lloyd_max, quantize

GOLD = os.path.join(os.path.dirname(__file__), "golden",
                    "gaussian_quantizer_max1960.txt")


def _max1960():
    rows = {}
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        b, thr, lev, mse = (f.strip() for f in line.split("|"))
        rows[int(b)] = ([float(t) for t in thr.split()],
                        [float(t) for t in lev.split()], float(mse))
    return rows


def test_one_bit_closed_form():
    levels, thr, mse = lloyd_max(1)
    assert abs(levels[1] - math.sqrt(2 / math.pi)) < 1e-15
    assert levels[0] == -levels[1] and thr.tolist() == [0.0]
    assert abs(mse - (1 - 2 / math.pi)) < 1e-14


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_matches_max_1960_table(bits):
    thr_ref, lev_ref, mse_ref = _max1960()[bits]
    levels, thr, mse = lloyd_max(bits)
    m = 2 ** (bits - 1)
    np.testing.assert_allclose(levels[m:], lev_ref, rtol=6e-4)
    np.testing.assert_allclose(thr[m:], thr_ref, rtol=6e-4)
    assert abs(mse / mse_ref - 1) < 6e-4


@pytest.mark.parametrize("bits", range(1, 9))
def test_optimality_conditions_by_quadrature(bits):
    levels, thr, mse = lloyd_max(bits)
    n = levels.size
    assert np.all(np.diff(levels) > 0) and np.all(np.diff(thr) > 0)
    np.testing.assert_array_equal(levels, -levels[::-1])
    # thresholds are midpoints of adjacent levels
    assert np.max(np.abs(thr - 0.5 * (levels[:-1] + levels[1:]))) < 1e-14
    # levels are centroids; checked with scipy quadrature on a few cells
    edges = np.concatenate([[-np.inf], thr, [np.inf]])
    for j in sorted({n // 2, n // 2 + 1, n - 2, n - 1} & set(range(n))):
        a, b = edges[j], edges[j + 1]
        mass = norm.cdf(b) - norm.cdf(a) if a < 0 else norm.sf(a) - norm.sf(b)
        first = integrate.quad(lambda x: x * norm.pdf(x), a, b, epsabs=1e-15,
                               epsrel=1e-13)[0]
        assert abs(first / mass - levels[j]) < 1e-9 * max(1.0, abs(levels[j]))
    # distortion by quadrature of (x - q(x))^2 over the positive half
    tot = 0.0
    for j in range(n // 2, n):
        a, b = edges[j], edges[j + 1]
        tot += integrate.quad(lambda x: (x - levels[j]) ** 2 * norm.pdf(x), a, b,
                              epsabs=1e-16, epsrel=1e-12, limit=200)[0]
    assert abs(2 * tot / mse - 1) < 1e-8


def test_high_rate_constant_panter_dite():
    c = [lloyd_max(b)[2] * 4.0 ** b for b in range(1, 9)]
    assert all(x < y for x, y in zip(c, c[1:]))
    pd = math.pi * math.sqrt(3) / 2
    assert c[-1] < pd and pd - c[-1] < 0.03


def test_float32_codebook():
    for b in range(1, 9):
        lv, th = codebook_f32(b)
        assert lv.dtype == np.float32 and th.dtype == np.float32
        assert th[th.size // 2] == 0.0


def test_quantize_decision_rule_float32():
    # two-bit table: thresholds -t, 0, t; exactly-on-threshold goes up
    _, th = codebook_f32(2)
    t = float(th[2])
    g = np.array([1.0], dtype=np.float32)
    c = np.array([[-10.0, -t, -1e-30, 0.0, 1e-30,
                   np.nextafter(np.float32(t), np.float32(0)), t, 10.0]])
    codes = quantize(c, g, np.array([2]))
    assert codes.tolist() == [[0, 1, 1, 2, 2, 2, 3, 3]]


def test_quantize_symmetry_and_zero_gain():
    rng = np.random.default_rng(3)
    c = rng.standard_normal((6, 64)).astype(np.float32)
    g = gains_f32(np.mean(c.astype(np.float64) ** 2, axis=1))
    for b in range(1, 9):
        bits = np.full(6, b)
        q1 = quantize(c, g, bits).astype(np.int64)
        q2 = quantize(-c, g, bits).astype(np.int64)
        assert np.array_equal(q1 + q2, np.full_like(q1, 2 ** b - 1))
    # gain 0: reconstructs to exactly zero
    z = np.zeros((1, 64))
    q = quantize(z, np.zeros(1, np.float32), np.array([3]))
    assert np.all(dequantize(q, np.zeros(1, np.float32), np.array([3])) == 0.0)
    # zero-bit bins: code 0, reconstruct 0
    q = quantize(c, g, np.zeros(6, np.int64))
    assert np.all(q == 0)
    assert np.all(dequantize(q, g, np.zeros(6, np.int64)) == 0.0)


def test_eight_bit_roundtrip_distortion():
    rng = np.random.default_rng(4)
    c = rng.standard_normal((64, 4096)) * 3.0
    g = gains_f32(np.mean(c ** 2, axis=1))
    bits = np.full(64, 8)
    r = dequantize(quantize(c, g, bits), g, bits)
    rel = np.mean((r - c) ** 2) / np.mean(c ** 2)
    assert abs(rel / lloyd_max(8)[2] - 1) < 0.05


def test_splitmix64_reference_values():
    # the generator's published reference sequence from state 0: outputs
    # 1..3 are the mix of states gamma, 2 gamma, 3 gamma
    from oracle import splitmix64
    gamma = 0x9E3779B97F4A7C15
    seq = [splitmix64(k * gamma % 2 ** 64) for k in range(3)]
    assert seq == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_rotation_is_orthogonal_and_block_hadamard():
    from scipy.linalg import hadamard
    from oracle import rotate, rotation_signs, unrotate
    for d in (64, 128, 256):
        eye = np.eye(d)
        R = rotate(eye).T                       # columns: R e_j
        assert np.max(np.abs(R @ R.T - eye)) < 1e-14
        s = rotation_signs()
        assert set(np.unique(s)) <= {-1.0, 1.0} and 0.3 < np.mean(s > 0) < 0.7
        # block structure: the same H_64 diag(s) / 8 on every 64-block
        blk = hadamard(64) * s / 8.0
        for b0 in range(0, d, 64):
            assert np.max(np.abs(R[b0:b0 + 64, b0:b0 + 64] - blk)) < 1e-15
        if d > 64:
            assert np.max(np.abs(R[:64, 64:])) == 0.0
        x = np.random.default_rng(d).standard_normal((3, d))
        assert np.max(np.abs(unrotate(rotate(x)) - x)) < 1e-13


def test_rotation_flattens_a_spike():
    # a single large coordinate spreads evenly: every rotated coordinate has
    # magnitude |x| / 8, so the heavy-tail ratio absmax / rms drops to 1
    from oracle import rotate
    x = np.zeros(128)
    x[5] = 8.0
    v = rotate(x)
    assert np.allclose(np.abs(v[:64]), 1.0) and np.all(v[64:] == 0.0)


# ---- the other quantizer backends of the page's comparison ----------------
def _normal_table():
    rows = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "normal_quantiles.txt")):
        if line.startswith("#") or not line.strip():
            continue
        p, z = line.split()
        rows[float(p)] = float(z)
    return rows


@pytest.mark.parametrize("bits", range(1, 9))
def test_uniform_quantizer_mse_on_uniform_input(bits):
    # a uniform quantizer with step D on U(-1, 1) has MSE D^2 / 12 (classic
    # result); checked by quantizing a fine grid of the interval
    from oracle import codebook
    lv, th = codebook(bits, "uniform")
    x = (np.arange(200000) + 0.5) / 100000.0 - 1.0
    y = lv[np.searchsorted(th, x, side="right")]
    step = 2.0 / 2 ** bits
    assert abs(np.mean((x - y) ** 2) / (step * step / 12.0) - 1) < 1e-3
    np.testing.assert_array_equal(lv, -lv[::-1])


def test_nf_levels_match_the_normal_table():
    from oracle import nf_levels
    z = _normal_table()
    for bits in (2, 3):
        n = 2 ** bits
        zmax = z[(n - 0.5) / n]
        upper = nf_levels(bits)[n // 2:]
        ref = [z[(k + 0.5) / n] / zmax for k in range(n // 2, n)]
        np.testing.assert_allclose(upper, ref, atol=2e-4)


@pytest.mark.parametrize("bits", range(1, 9))
def test_nf_levels_sit_at_equal_probability_centres(bits):
    # Phi(level * z_max) = (k + 1/2) / 2^b, with Phi from the oracle's own
    # complementary error function (independent of the quantile routine)
    from oracle import nf_levels
    from oracle.tact_oracle import _upper_tail
    n = 2 ** bits
    lv = nf_levels(bits)
    # z_max is the quantile at (n - 1/2) / n: solve it by bisection on erfc
    lo, hi = 0.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if 1.0 - _upper_tail(mid) < (n - 0.5) / n:
            lo = mid
        else:
            hi = mid
    zmax = 0.5 * (lo + hi)
    cdf = 1.0 - _upper_tail(lv * zmax)
    np.testing.assert_allclose(cdf, (np.arange(n) + 0.5) / n, atol=1e-12)


def test_lloyd_max_beats_the_other_backends_at_low_rate():
    # at 1-3 bits the Gaussian Lloyd-Max table with the RMS gain beats both
    # absmax-scaled grids on Gaussian bins (their outer levels sit at the
    # bin's extreme value, far in the tail); from 4 bits on, NormalFloat's
    # per-vector range catches up, so the comparison stops at 3
    from oracle import gains_absmax_f32
    rng = np.random.default_rng(11)
    c = rng.standard_normal((2000, 128))
    g_rms = gains_f32(np.mean(c ** 2, axis=1))
    g_abs = gains_absmax_f32(c)
    for b in (1, 2, 3):
        bits = np.full(2000, b)
        e = {}
        for kind, g in (("lloyd_max", g_rms), ("uniform", g_abs), ("nf", g_abs)):
            r = dequantize(quantize(c, g, bits, kind=kind), g, bits, kind=kind)
            e[kind] = np.mean((r - c) ** 2)
        assert e["lloyd_max"] < e["uniform"] and e["lloyd_max"] < e["nf"], (b, e)


def test_heavy_tails_hurt_absmax_backends_most():
    # the page's explanation of its quantizer comparison: with heavy-tailed
    # coefficients (Student-t, 3 degrees of freedom) the absmax-scaled grids
    # waste their range, while gain-shape SQ with the rotation keeps its
    # distortion near the Gaussian value
    from oracle import gains_absmax_f32
    rng = np.random.default_rng(12)
    c = rng.standard_t(3, size=(2000, 128))
    bits = np.full(2000, 1)
    g_rms = gains_f32(np.mean(c ** 2, axis=1))
    r = dequantize(quantize(c, g_rms, bits, "hadamard"), g_rms, bits, "hadamard")
    e_lm = np.mean((r - c) ** 2) / np.mean(c ** 2)
    for kind in ("uniform", "nf"):
        g = gains_absmax_f32(c)
        r = dequantize(quantize(c, g, bits, kind=kind), g, bits, kind=kind)
        assert np.mean((r - c) ** 2) / np.mean(c ** 2) > 1.2 * e_lm


def test_absmax_gain_is_taken_after_the_rotation():
    # The uniform and NormalFloat backends scale by the largest |value| of
    # the vector they quantize, which with the rotation on is R u.  Two hand
    # cases fix the order.  (1) A spike 8 e_5 in the first 64-block: every
    # coordinate of R(8 e_5) = H_64 diag(s) 8 e_5 / 8 is s_5 H[j][5] = +-1,
    # so the rotated gain is 1 while the unrotated one is 8.  (2) The
    # vector c_j = s_j (-1)^popcount(j & 9) (all +-1) is R^T (8 e_9): its
    # rotated image is 8 at coordinate 9 and 0 elsewhere, so the rotated
    # gain is 8 while the unrotated one is 1.  The second 64-block carries
    # the same pattern shifted, so each block is rotated on its own.
    from oracle import gains_absmax_f32, rotation_signs
    s = rotation_signs()
    spike = np.zeros((2, 128))
    spike[0, 5] = 8.0
    spike[1, 64 + 5] = 8.0
    np.testing.assert_array_equal(gains_absmax_f32(spike, "none"), [8.0, 8.0])
    np.testing.assert_array_equal(gains_absmax_f32(spike, "hadamard"), [1.0, 1.0])
    par = np.array([(-1.0) ** bin(j & 9).count("1") for j in range(64)])
    flat = np.zeros((2, 128))
    flat[0, :64] = s * par
    flat[1, 64:] = s * par
    flat[1, :64] = 0.5 * s * par          # a second block below the first
    np.testing.assert_array_equal(gains_absmax_f32(flat, "none"), [1.0, 1.0])
    np.testing.assert_array_equal(gains_absmax_f32(flat, "hadamard"), [8.0, 8.0])
    # and the quantizer decides on the rotated vector scaled by that gain:
    # at 1 bit the uniform grid has levels +-1/2 and its threshold at 0, so
    # the codes of the spike are the signs of s_5 H[j][5]
    from oracle import quantize
    codes = quantize(spike[:1, :64], np.float32([1.0]), np.array([1]), "hadamard",
                     kind="uniform")
    hcol = np.array([(-1.0) ** bin(j & 5).count("1") for j in range(64)])
    np.testing.assert_array_equal(codes[0], (s[5] * hcol > 0).astype(np.uint8))
