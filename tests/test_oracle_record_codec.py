"""Pins of the oracle's record format (hand-derived fixture) and whole-codec
properties: occupancy, pack/unpack inverse, lossless transform at full rate,
and the Gaussian heavy-tail reference statistic."""
import os

import numpy as np
import pytest
import torch

from oracle import (Params, absmax_to_std, allocate_bits, bin_variance,
                    compress, dct3_forward, decompress, gains_f32, mse,
                    occupancy_bits, pack_record, quantize, record_layout,
                    total_bits, unpack_record)
from tact_inputs import WORKLOADS, generate_unit

GOLD = os.path.join(os.path.dirname(__file__), "golden", "record_hand_cases.txt")


def _fixture():
    cases = {}
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        case, region, hexs = line.split()
        cases.setdefault(case, {})[region] = bytes.fromhex(hexs)
    return cases


@pytest.mark.parametrize("case", ["A", "B"])
def test_record_matches_hand_fixture(case):
    p = Params(1, 1, 2, 1, 64, budget_bits=1, max_bits=2)
    lay = record_layout(p)
    assert (lay["gains"], lay["bits"], lay["groups"], lay["codes"], lay["size"]) == \
        (0, 256, 512, 768, 1024)
    j = np.arange(64)
    if case == "A":
        bits = np.array([2, 0])
        gains = np.array([1.5, 0.25], np.float32)
        codes = np.stack([j % 4, np.zeros(64, int)])
    else:
        bits = np.array([1, 1])
        gains = np.array([2.0, 0.5], np.float32)
        codes = np.stack([j % 2, (j < 8).astype(int)])
    rec = pack_record(codes.reshape(1, 1, 2, 1, 64), gains, bits, p)
    exp = _fixture()[case]
    assert bytes(rec[0:8]) == exp["gains"]
    assert bytes(rec[256:258]) == exp["bits"]
    assert bytes(rec[512:516]) == exp["groups"]
    assert bytes(rec[768:784]) == exp["codes"]
    assert not rec[8:256].any() and not rec[784:].any()
    c2, g2, b2 = unpack_record(rec, p)
    assert np.array_equal(c2.reshape(2, 64)[bits > 0], codes[bits > 0])
    assert np.array_equal(g2.ravel(), gains) and np.array_equal(b2.ravel(), bits)


def test_group_index_spans_groups():
    p = Params(1, 1, 65, 2, 64, budget_bits=1, max_bits=2)   # 130 bins, T = 130
    bits = np.ones(130, int)
    bits[0], bits[129] = 2, 0
    codes = np.zeros((130, 64), int)
    rec = pack_record(codes.reshape(p.shape), np.ones(130, np.float32), bits, p)
    lay = record_layout(p)
    grp = rec[lay["groups"]:lay["groups"] + 12].view("<u4").tolist()
    assert grp == [0, 65, 129]   # planes before bins 0, 64, 128 (worked by hand)


def test_pack_unpack_inverse_random():
    rng = np.random.default_rng(0)
    p = Params(2, 3, 4, 2, 128, budget_bits=3, max_bits=8)
    var = np.exp(rng.normal(0, 3, p.n_bins))
    bits = allocate_bits(var, total_bits(p), 8)
    codes = rng.integers(0, 256, (p.n_bins, 128)) & ((1 << bits[:, None]) - 1)
    codes[bits == 0] = 0
    gains = rng.random(p.n_bins).astype(np.float32)
    rec = pack_record(codes.reshape(p.shape), gains, bits, p)
    assert rec.size == record_layout(p)["size"]
    c, g, b = unpack_record(rec, p)
    assert np.array_equal(c.reshape(p.n_bins, 128), codes)
    assert np.array_equal(b.ravel(), bits) and np.array_equal(g.ravel(), gains)


def test_code_bytes_and_page_occupancy():
    p = Params(4, 8, 8, 2, 64, budget_bits=1, max_bits=3)
    lay = record_layout(p)
    assert lay["code_bytes"] == p.n_bins * 1 * 64 // 8
    bits = np.array([3, 0, 1, 2])
    assert occupancy_bits(bits, 64) == (3 + 1 + 2) * 64 + 3 * 32


def _tiny_unit(kv=0):
    wl = WORKLOADS["tiny"]
    return generate_unit(wl, 0, 0, kv).numpy().astype(np.float64)


def test_full_rate_distortion_is_lloyd_max_8bit():
    # Gaussian input, every bin at 8 bits: relative distortion ~ mse_8 (4.1e-5)
    x = np.random.default_rng(2).standard_normal((4, 8, 8, 2, 64))
    p = Params(4, 8, 8, 2, 64, budget_bits=8, max_bits=8)
    rec = compress(x, p)
    y = decompress(rec, p, out_dtype=None)
    rel = np.mean((y - x) ** 2) / np.mean(x ** 2)
    assert 2e-5 < rel < 1e-4


def test_heavy_tail_channel_clips_at_full_rate():
    # with the identity rotation a x8 channel lands far outside the 8-bit
    # table's range (largest level ~4.6): clipping dominates the distortion
    x = _tiny_unit()
    p = Params(4, 8, 8, 2, 64, budget_bits=8, max_bits=8)
    y = decompress(compress(x, p, rotation="none"), p, out_dtype=None, rotation="none")
    rel = np.mean((y - x) ** 2) / np.mean(x ** 2)
    assert rel > 1e-3


def test_tiny_roundtrip_budget_and_distortion():
    x = _tiny_unit()
    p = Params(4, 8, 8, 2, 64, budget_bits=1, max_bits=3)
    rec = compress(x, p)
    _, g, b = unpack_record(rec, p)
    assert b.sum() == total_bits(p) and b.max() <= 3
    y = decompress(rec, p, out_dtype="f32")
    rel = np.mean((y - x) ** 2) / np.mean(x ** 2)
    # 1 bit per entry on a strongly correlated field: far below the energy
    assert 0 < rel < 0.25
    # more budget, less distortion
    p2 = Params(4, 8, 8, 2, 64, budget_bits=2, max_bits=3)
    y2 = decompress(compress(x, p2), p2, out_dtype="f32")
    assert np.mean((y2 - x) ** 2) < np.mean((y - x) ** 2)


def test_zero_bit_bins_reconstruct_zero_coefficients():
    x = _tiny_unit(1)
    p = Params(4, 8, 8, 2, 64, budget_bits=1, max_bits=3)
    c = dct3_forward(x)
    var = bin_variance(c)
    bits = allocate_bits(var, total_bits(p), 3).reshape(var.shape)
    q = quantize(c, gains_f32(var), bits)
    assert np.all(q[bits == 0] == 0)


def test_gaussian_heavy_tail_reference():
    # the page's Gaussian reference for median absmax/std at d = 256 is 3.01
    rng = np.random.default_rng(1)
    c = rng.standard_normal((4000, 256))
    assert abs(np.median(absmax_to_std(c)) - 3.01) < 0.03


def test_generator_is_deterministic_and_shaped():
    wl = WORKLOADS["tiny"]
    a = generate_unit(wl, 0, 0, 0)
    b = generate_unit(wl, 0, 0, 0)
    assert a.dtype == torch.float32 and tuple(a.shape) == (4, 8, 8, 2, 64)
    assert torch.equal(a, b)
    assert not torch.equal(a, generate_unit(wl, 0, 0, 1))


def test_ablations_transform_and_allocation_order():
    # on a field correlated along all three axes, dropping axes or adaptive
    # allocation can only lose (the page's ablation ordering); uniform
    # allocation gives every bin the budget
    from oracle import allocate_uniform, roundtrip
    x = np.random.default_rng(5).standard_normal((8, 8, 8, 1, 64))
    for ax, rho in ((0, 0.95), (1, 0.95), (2, 0.95)):
        for i in range(1, x.shape[ax]):
            cur = np.take(x, i, axis=ax)
            prev = np.take(x, i - 1, axis=ax)
            idx = [slice(None)] * x.ndim
            idx[ax] = i
            x[tuple(idx)] = rho * prev + np.sqrt(1 - rho * rho) * cur
    p = Params(8, 8, 8, 1, 64, budget_bits=1, max_bits=8)
    e3 = mse(roundtrip(x, p, None)[0], x)
    e1 = mse(roundtrip(x, p, None, axes=(0,))[0], x)
    eu = mse(roundtrip(x, p, None, alloc="uniform")[0], x)
    assert e3 < e1 and e3 < eu
    assert allocate_uniform(np.zeros(7), 3).tolist() == [3] * 7


def test_rotation_removes_heavy_tail_clipping_at_full_rate():
    # the x8 channel that clips without rotation is spread by the shared
    # rotation; distortion at 8 bits falls back near the Lloyd-Max level
    from oracle import roundtrip
    x = _tiny_unit()
    p = Params(4, 8, 8, 2, 64, budget_bits=8, max_bits=8)
    e_none = np.mean((roundtrip(x, p, None, rotation="none")[0] - x) ** 2) / np.mean(x ** 2)
    e_rot = np.mean((roundtrip(x, p, None)[0] - x) ** 2) / np.mean(x ** 2)
    assert e_rot < 1e-4 < e_none
