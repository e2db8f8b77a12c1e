"""Decoding of records whose group index or bit widths are inconsistent.

The record layout (include/tact.h) stores, besides the bit widths b_i, a group
index with the first bit-plane of every 64th bin; decoding locates each bin's
planes from both.  Every record tact_compress writes is consistent.  For one
that is not, the library promises unspecified values but no access outside
the record, the output or the workspace: widths above max_bits and planes
past the record's T planes decode as zero, and every code-word load is
range-checked.  These tests corrupt real records in three ways and check that
decompression (plane-kernel and per-axis paths) and fused attention return
normally with finite output; an unmodified record is the control.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.device_count() > 0:
    import kv_cache_compression_tact_amd as tact


def say(*a):
    print(*a, flush=True)


def _align256(n):
    return (n + 255) // 256 * 256


def _offsets(g):
    """Byte offsets of the bit widths and the group index in one record."""
    nb = g.S * g.H * g.W * g.kv_heads
    off_bits = _align256(4 * nb)
    off_groups = off_bits + _align256(nb)
    return nb, off_bits, off_groups, (nb + 63) // 64


def _records(g, n, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((n,) + g.unit_shape, generator=gen, dtype=torch.float32).to(g.dtype).cuda()
    return tact.compress(x, g.budget_bits, g.max_bits)


def _corrupt(rec, g, how):
    nb, ob, og, ng = _offsets(g)
    r = rec.clone()
    if how == "groups_huge":
        r[:, og:og + 4 * ng] = torch.tensor([0xF0, 0xFF, 0xFF, 0xFF], dtype=torch.uint8,
                                            device=r.device).repeat(ng)
    elif how == "groups_zero":
        r[:, og:og + 4 * ng] = 0
    elif how == "bits_wide":
        r[:, ob:ob + nb:3] = 200
    return r


CASES = ["none", "groups_huge", "groups_zero", "bits_wide"]
GEOMS = [
    (4, 8, 8, 2, 64, 2, 8),      # plane kernels
    (3, 17, 23, 2, 128, 2, 8),   # plane kernels, ragged 32-wide planes
    (3, 5, 40, 1, 128, 2, 8),    # W beyond 32: per-axis kernels
]


@pytest.mark.parametrize("geo", GEOMS)
@pytest.mark.parametrize("how", CASES)
def test_decompress_inconsistent_record(geo, how):
    S, H, W, hk, d, budget, bmax = geo
    say("decompress", geo, how)
    g = tact.Geometry(S, H, W, hk, d, budget, max_bits=bmax, dtype=torch.float32)
    rec = _records(g, 2, seed=31)
    ref = tact.decompress(rec, g)
    out = tact.decompress(_corrupt(rec, g, how), g)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    if how == "none":
        assert torch.equal(out, ref)


@pytest.mark.parametrize("how", CASES)
def test_attend_inconsistent_record(how):
    S, H, W, hk, d, budget, bmax = 4, 8, 8, 2, 128, 2, 8
    say("attend", how)
    g = tact.Geometry(S, H, W, hk, d, budget, max_bits=bmax, dtype=torch.float32)
    rec = _records(g, 4, seed=32)
    k, v = rec[0::2].contiguous(), rec[1::2].contiguous()
    q = torch.from_numpy(np.random.default_rng(33).standard_normal((2, 8, d)).astype(np.float32)).cuda()
    ref_out, ref_lse = tact.attend(k, v, g, q)
    out, lse = tact.attend(_corrupt(k, g, how), _corrupt(v, g, how), g, q)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    if how == "none":
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
