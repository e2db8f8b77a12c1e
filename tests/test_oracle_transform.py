"""Pins of the oracle's transform and variance against facts outside it:
scipy's orthonormal DCT-II (an independent library routine), orthonormality,
Parseval, exact inversion, and closed-form inputs."""
import math

import numpy as np
import pytest
import scipy.fft

from oracle import (Params, bin_variance, bf16_bits, dct2_matrix, dct3_forward,
                    dct3_inverse, round_to_bf16)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 14, 16, 24, 32, 60, 64])
def test_dct_matrix_orthonormal(n):
    c = dct2_matrix(n)
    assert np.max(np.abs(c @ c.T - np.eye(n))) < 1e-14


@pytest.mark.parametrize("n", [1, 2, 4, 14, 24, 64])
def test_dct_matrix_matches_scipy(n):
    x = np.random.default_rng(n).standard_normal((n, 5))
    ref = scipy.fft.dct(x, type=2, norm="ortho", axis=0)
    assert np.max(np.abs(dct2_matrix(n) @ x - ref)) < 1e-13


@pytest.mark.parametrize("shape", [(4, 8, 8, 2, 8), (3, 5, 7, 1, 4), (6, 14, 14, 2, 2)])
def test_dct3_matches_scipy_dctn(shape):
    x = np.random.default_rng(1).standard_normal(shape)
    ref = scipy.fft.dctn(x, type=2, norm="ortho", axes=(0, 1, 2))
    assert np.max(np.abs(dct3_forward(x) - ref)) < 1e-12
    back = scipy.fft.idctn(ref, type=2, norm="ortho", axes=(0, 1, 2))
    assert np.max(np.abs(dct3_inverse(ref) - back)) < 1e-12


@pytest.mark.parametrize("axes", [(0,), (1, 2), (0, 2), (0, 1, 2)])
def test_axis_subsets_match_scipy(axes):
    x = np.random.default_rng(2).standard_normal((4, 6, 5, 2, 3))
    ref = scipy.fft.dctn(x, type=2, norm="ortho", axes=axes)
    assert np.max(np.abs(dct3_forward(x, axes) - ref)) < 1e-12
    assert np.max(np.abs(dct3_inverse(ref, axes) - x)) < 1e-12


def test_parseval_and_variance_sum():
    x = np.random.default_rng(3).standard_normal((4, 8, 8, 2, 64)) * 3.0
    c = dct3_forward(x)
    assert abs(np.sum(c * c) / np.sum(x * x) - 1.0) < 1e-12
    var = bin_variance(c)
    assert var.shape == (4, 8, 8, 2)
    # d * sum of per-bin variances is the total energy
    assert abs(64 * var.sum() / np.sum(x * x) - 1.0) < 1e-12


def test_variance_is_second_moment_over_head_dim():
    c = np.zeros((1, 1, 1, 2, 4))
    c[0, 0, 0, 0] = [1.0, -1.0, 1.0, -1.0]      # mean 0, second moment 1
    c[0, 0, 0, 1] = [2.0, 2.0, 2.0, 2.0]        # mean 2, second moment 4
    v = bin_variance(c)
    assert v[0, 0, 0, 0] == 1.0 and v[0, 0, 0, 1] == 4.0


def test_constant_volume_only_dc():
    S, H, W = 4, 6, 8
    x = np.full((S, H, W, 1, 3), 2.5)
    c = dct3_forward(x)
    assert abs(c[0, 0, 0, 0, 0] - 2.5 * math.sqrt(S * H * W)) < 1e-12
    c[0, 0, 0] = 0.0
    assert np.max(np.abs(c)) < 1e-12


def test_separable_cosine_lands_in_one_bin():
    S, H, W = 5, 6, 7
    ks, kh, kw = 2, 5, 3
    # x[s,h,w] = cos(pi(2s+1)ks/2S) cos(pi(2h+1)kh/2H) cos(pi(2w+1)kw/2W)
    s = np.cos(np.pi * (2 * np.arange(S) + 1) * ks / (2 * S))
    h = np.cos(np.pi * (2 * np.arange(H) + 1) * kh / (2 * H))
    w = np.cos(np.pi * (2 * np.arange(W) + 1) * kw / (2 * W))
    x = np.einsum("a,b,c->abc", s, h, w)[..., None, None]
    c = dct3_forward(x)
    # the basis vector with k >= 1 has norm sqrt(N/2)
    expect = math.sqrt(S / 2) * math.sqrt(H / 2) * math.sqrt(W / 2)
    assert abs(c[ks, kh, kw, 0, 0] - expect) < 1e-12
    c[ks, kh, kw] = 0.0
    assert np.max(np.abs(c)) < 1e-12


def test_inverse_is_exact_on_bf16_input():
    # quantization bypassed ("infinite bits"): the transform is lossless,
    # so rounding the fp64 reconstruction to bf16 returns the input bits.
    rng = np.random.default_rng(4)
    x = round_to_bf16(rng.standard_normal((4, 8, 8, 2, 64)) * 10.0)
    y = round_to_bf16(dct3_inverse(dct3_forward(x)))
    assert np.array_equal(bf16_bits(x), bf16_bits(y))


def test_round_to_bf16_matches_nearest_even():
    # bf16 has 8 significant bits: between 1 and 2 the spacing is 2^-7
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-30,
                     -(1.0 + 2**-8), 3.0 + 2**-7, 1.0 + 2**-8 - 2**-40])
    exp = np.array([1.0, 1.0, 1.0 + 2 * 2**-7, 1.0 + 2**-7, -1.0, 3.0,
                    1.0])
    assert np.array_equal(round_to_bf16(vals), exp)
    assert bf16_bits(np.array([1.0]))[0] == 0x3F80
    assert bf16_bits(np.array([-2.0]))[0] == 0xC000


def test_params_geometry():
    p = Params(64, 24, 24, 8, 128, budget_bits=1)
    assert p.n_bins == 294912 and p.n_entries == 37748736
