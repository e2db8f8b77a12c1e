"""Decoding fused into attention on the GPU against the oracle's attention
over the decoded cache (records written by the oracle, so no input of the
comparison comes from the HIP path).

Error bound.  The kernel works in fp32: per-bin projections (sums of
head_dim products), an inverse 3-D DCT of the score field (sums of at most
64 terms per axis, split-fp16 products good to 2^-22), the softmax, a
forward 3-D DCT of the probabilities and a sum over the coded V bins.  Each
stage's rounding errors add up like a random walk, about sqrt(n) * 2^-24 of
the magnitudes it sums (n <= 256 terms), so the scores carry an absolute
error of about 1e-6 of the largest |score|, which moves lse by as much and
every probability by that relative amount (measured: at most 6.4e-7 in
these units).  The bars, ten times that:
  |lse - lse_ref| <= 1e-5 * (1 + max_t |score_t|)
  max_j |out_j - out_ref_j| <= 1e-5 * (1 + max_t |score_t|) * RMS(V of the head)
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from tact_inputs import WORKLOADS, generate_unit

pytestmark = pytest.mark.gpu

if torch.cuda.device_count() > 0:
    import kv_cache_compression_tact_amd as tact


def say(*a):
    print(*a, flush=True)


def _field(shape, seed):
    """A correlated field of the unit shape (fp64, CPU)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    for ax, rho in ((0, 0.9), (1, 0.85), (2, 0.8)):
        for i in range(1, x.shape[ax]):
            idx = [slice(None)] * x.ndim
            prev = list(idx)
            idx[ax] = i
            prev[ax] = i - 1
            x[tuple(idx)] = rho * x[tuple(prev)] + math.sqrt(1 - rho * rho) * x[tuple(idx)]
    return x


def _check(krec, vrec, p, q, scale, rotation, axes=(0, 1, 2), out=None, lse=None):
    """Compare GPU (out, lse) of every pair with the oracle."""
    worst = 0.0
    for u in range(q.shape[0]):
        o_ref, l_ref = O.attend(krec[u], vrec[u], p, q[u], scale, axes, rotation)
        K = O.decompress(krec[u], p, None, axes, rotation)
        V = O.decompress(vrec[u], p, None, axes, rotation)
        rep = q.shape[1] // p.kv_heads
        for r in range(q.shape[1]):
            h = r // rep
            smax = np.max(np.abs(scale * (K[:, :, :, h, :].reshape(-1, p.head_dim) @ q[u, r])))
            vrms = math.sqrt(np.mean(V[:, :, :, h, :] ** 2))
            e_l = abs(float(lse[u, r]) - l_ref[r])
            e_o = float(np.max(np.abs(out[u, r] - o_ref[r])))
            assert e_l <= 1e-5 * (1 + smax), (u, r, e_l, smax)
            assert e_o <= 1e-5 * (1 + smax) * vrms, (u, r, e_o, smax, vrms)
            worst = max(worst, e_o / ((1 + smax) * vrms), e_l / (1 + smax))
    say(f"  worst relative error {worst:.2e}")


ATT_GEOMS = [
    # (S, H, W, kv_heads, head_dim, budget, bmax, q_heads, rotation)
    (4, 8, 8, 2, 64, 1, 3, 4, "hadamard"),          # the tiny unit shape
    (5, 7, 9, 3, 64, 2, 8, 6, "hadamard"),          # ragged everywhere
    (3, 14, 14, 1, 128, 1, 8, 7, "hadamard"),       # 7 query heads per kv head
    (2, 5, 3, 2, 256, 4, 8, 32, "hadamard"),        # 16 per kv head, head_dim 256
    (33, 3, 2, 1, 128, 3, 5, 1, "none"),            # S beyond 32, no rotation
    (3, 17, 23, 2, 128, 2, 8, 4, "hadamard"),       # H, W beyond 16
    (2, 2, 40, 1, 64, 1, 8, 2, "hadamard"),         # W beyond 32
    (4, 6, 5, 2, 64, 2, 8, 6, "hadamard"),          # 3 per kv head (one padded head)
    (3, 5, 7, 1, 256, 2, 6, 5, "none"),             # 5 per kv head (three padded heads)
    (2, 4, 4, 2, 128, 8, 8, 8, "hadamard"),         # every bin coded at 8 bits
]


@pytest.mark.parametrize("geo", ATT_GEOMS)
def test_attend_matches_oracle(geo):
    S, H, W, hk, d, budget, bmax, qh, rot = geo
    say("attend", geo)
    p = O.Params(S, H, W, hk, d, budget, bmax)
    g = tact.Geometry(S, H, W, hk, d, budget, max_bits=bmax,
                      rotation=tact.ROTATION_HADAMARD if rot == "hadamard" else tact.ROTATION_NONE)
    pairs = 2
    krec = np.stack([O.compress(_field(p.shape, 10 * u), p, rotation=rot) for u in range(pairs)])
    vrec = np.stack([O.compress(_field(p.shape, 10 * u + 1), p, rotation=rot) for u in range(pairs)])
    q = np.random.default_rng(7).standard_normal((pairs, qh, d)).astype(np.float32) * 2.0
    scale = 1.0 / math.sqrt(d)
    out, lse = tact.attend(torch.from_numpy(krec).cuda(), torch.from_numpy(vrec).cuda(), g,
                           torch.from_numpy(q).cuda(), scale)
    torch.cuda.synchronize()
    _check(krec, vrec, p, q.astype(np.float64), scale, rot,
           out=out.cpu().numpy().astype(np.float64), lse=lse.cpu().numpy().astype(np.float64))


def _random_att_geometries(n, seed):
    # seeded shapes: every field axis from 1 to 64 / 32 / 40, 1..3 kv heads,
    # every head_dim, 1..8 query heads per kv head, both rotations
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        S, H, W = int(rng.integers(1, 65)), int(rng.integers(1, 33)), int(rng.integers(1, 41))
        hk, d = int(rng.integers(1, 4)), int(rng.choice([64, 128, 256]))
        if S * H * W * hk * d > 60000:
            continue
        bmax = int(rng.integers(1, 9))
        out.append((S, H, W, hk, d, int(rng.integers(1, bmax + 1)), bmax,
                    hk * int(rng.integers(1, 9)), "hadamard" if rng.random() < 0.8 else "none"))
    return out


@pytest.mark.parametrize("geo", _random_att_geometries(6, 4242))
def test_attend_random_geometries(geo):
    test_attend_matches_oracle(geo)


@pytest.mark.parametrize("quant", [1, 2])
def test_attend_quantizer_backends(quant):
    # records coded with the uniform or NormalFloat table (absmax gains)
    S, H, W, hk, d = 4, 6, 5, 2, 128
    name = O.QUANTIZERS[quant]
    p = O.Params(S, H, W, hk, d, 2, 8)
    g = tact.Geometry(S, H, W, hk, d, 2, quantizer=quant)
    krec = O.compress(_field(p.shape, 21), p, quantizer=name)[None]
    vrec = O.compress(_field(p.shape, 22), p, quantizer=name)[None]
    q = np.random.default_rng(23).standard_normal((1, 8, d)).astype(np.float32)
    out, lse = tact.attend(torch.from_numpy(krec).cuda(), torch.from_numpy(vrec).cuda(), g,
                           torch.from_numpy(q).cuda(), 0.1)
    worst = 0.0
    o_ref, l_ref = O.attend(krec[0], vrec[0], p, q[0].astype(np.float64), 0.1, quantizer=name)
    V = O.decompress(vrec[0], p, None, quantizer=name)
    o, l = out.cpu().numpy()[0], lse.cpu().numpy()[0]
    for r in range(8):
        vrms = math.sqrt(np.mean(V[:, :, :, r // 4, :] ** 2))
        assert abs(l[r] - l_ref[r]) <= 1e-5 * (1 + abs(l_ref[r]))
        assert np.max(np.abs(o[r] - o_ref[r])) <= 1e-5 * vrms * (1 + abs(l_ref[r]))


@pytest.mark.parametrize("axes", [(0, 2), (0, 1), (1, 2), (1,), ()])
def test_attend_axis_subset(axes):
    # records coded with a subset of the axes, or with none: the field
    # transforms follow (the last inverse pass, which also yields the scores'
    # maximum, and the last forward pass, which writes the field out, are
    # then other axes than S and W)
    S, H, W, hk, d = 6, 5, 7, 2, 64
    p = O.Params(S, H, W, hk, d, 2, 8)
    g = tact.Geometry(S, H, W, hk, d, 2, axes=sum(1 << a for a in axes))
    krec = O.compress(_field(p.shape, 3), p, axes=axes)[None]
    vrec = O.compress(_field(p.shape, 4), p, axes=axes)[None]
    q = np.random.default_rng(8).standard_normal((1, 4, d)).astype(np.float32)
    out, lse = tact.attend(torch.from_numpy(krec).cuda(), torch.from_numpy(vrec).cuda(), g,
                           torch.from_numpy(q).cuda(), 0.125)
    _check(krec, vrec, p, q.astype(np.float64), 0.125, "hadamard", axes,
           out=out.cpu().numpy().astype(np.float64), lse=lse.cpu().numpy().astype(np.float64))


def test_attend_zero_budget_is_uniform_over_zero_values():
    # budget 0: no bin is coded, every decoded key and value is 0, so the
    # softmax is uniform (lse = log of the token count) and the output is 0
    S, H, W, hk, d = 3, 4, 5, 1, 64
    p = O.Params(S, H, W, hk, d, 0, 8)
    g = tact.Geometry(S, H, W, hk, d, 0)
    rec = O.compress(_field(p.shape, 5), p)[None]
    q = torch.randn(1, 2, d).cuda()
    out, lse = tact.attend(torch.from_numpy(rec).cuda(), torch.from_numpy(rec).cuda(), g, q)
    assert torch.all(out == 0)
    assert torch.allclose(lse.cpu(), torch.full((1, 2), math.log(S * H * W)), atol=1e-6)


@pytest.mark.parametrize("name", ["ct4b", "ct7b", "ct32b", "video"])
def test_attend_full_size_pair(name):
    """One layer's K and V at the workload's full unit size (the largest field
    that fits: 64 x 24 x 24 for ct32b), records written by the oracle."""
    wl = WORKLOADS[name]
    say("attend full size", name)
    p = O.Params(*wl.unit_shape, 1, wl.max_bits)
    g = tact.Geometry(*wl.unit_shape, 1, max_bits=wl.max_bits)
    k = generate_unit(wl, 0, 0, 0).float().numpy().astype(np.float64)
    v = generate_unit(wl, 0, 0, 1).float().numpy().astype(np.float64)
    krec, vrec = O.compress(k, p)[None], O.compress(v, p)[None]
    qh = 4 * p.kv_heads
    q = np.random.default_rng(9).standard_normal((1, qh, p.head_dim)).astype(np.float32)
    scale = 1.0 / math.sqrt(p.head_dim)
    out, lse = tact.attend(torch.from_numpy(krec).cuda(), torch.from_numpy(vrec).cuda(), g,
                           torch.from_numpy(q).cuda(), scale)
    _check(krec, vrec, p, q.astype(np.float64), scale, "hadamard",
           out=out.cpu().numpy().astype(np.float64), lse=lse.cpu().numpy().astype(np.float64))


def test_attend_matches_attention_over_gpu_decompressed_cache():
    # the fused path agrees with decompressing to fp32 on the GPU and running
    # plain attention there (same records, both paths of the library)
    S, H, W, hk, d = 8, 6, 6, 2, 128
    g = tact.Geometry(S, H, W, hk, d, 2, dtype=torch.float32)
    x = torch.from_numpy(np.stack([_field((S, H, W, hk, d), s) for s in range(4)])).float().cuda()
    rec = tact.compress(x, 2)
    dec = tact.decompress(rec, g).double()
    q = torch.randn(2, 8, d, dtype=torch.float32).cuda()
    out, lse = tact.attend(rec[0::2].contiguous(), rec[1::2].contiguous(), g, q)
    for u in range(2):
        for r in range(8):
            h = r // 4
            k = dec[2 * u][:, :, :, h, :].reshape(-1, d)
            v = dec[2 * u + 1][:, :, :, h, :].reshape(-1, d)
            s = (k @ q[u, r].double()) / math.sqrt(d)
            ref_l = torch.logsumexp(s, 0)
            ref_o = torch.softmax(s, 0) @ v
            assert abs(lse[u, r].item() - ref_l.item()) < 1e-5 * (1 + s.abs().max().item())
            assert (out[u, r].double() - ref_o).abs().max().item() < 1e-5 * (
                1 + s.abs().max().item()) * v.pow(2).mean().sqrt().item()
