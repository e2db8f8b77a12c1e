"""Pins of the oracle's attention over a decoded visual cache: torch's own
scaled-dot-product attention on the same decoded tensors, the merge rule of
the log-sum-exp with a disjoint token set, and the transform identities the
fused GPU kernel relies on (scores are the inverse 3-D DCT of per-bin
projections; the output is a sum over bins weighted by the forward DCT of
the probabilities)."""
import numpy as np
import pytest
import torch

from oracle import (Params, attend, compress, dct3_forward, dct3_inverse,
                    decompress)


def _pair(p, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((2,) + p.shape)
    # some smoothness so that the allocation is uneven
    x = np.cumsum(x, axis=1) / np.sqrt(np.arange(1, p.S + 1))[None, :, None, None, None, None]
    return compress(x[0], p), compress(x[1], p)


@pytest.mark.parametrize("geo,qh", [((3, 5, 4, 2, 64, 2, 8), 4), ((2, 3, 7, 1, 128, 1, 8), 3)])
def test_matches_torch_sdpa(geo, qh):
    p = Params(*geo)
    kr, vr = _pair(p, 1)
    q = np.random.default_rng(2).standard_normal((qh, p.head_dim))
    scale = 1.0 / np.sqrt(p.head_dim)
    out, lse = attend(kr, vr, p, q, scale)
    K = torch.from_numpy(decompress(kr, p, None))
    V = torch.from_numpy(decompress(vr, p, None))
    n = p.S * p.H * p.W
    rep = qh // p.kv_heads
    for r in range(qh):
        h = r // rep
        k = K[:, :, :, h, :].reshape(1, 1, n, p.head_dim)
        v = V[:, :, :, h, :].reshape(1, 1, n, p.head_dim)
        qq = torch.from_numpy(q[r]).reshape(1, 1, 1, p.head_dim)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=scale)
        np.testing.assert_allclose(out[r], ref.reshape(-1).numpy(), rtol=1e-12, atol=1e-12)
        s = scale * (k.reshape(n, -1) @ qq.reshape(-1))
        assert abs(lse[r] - torch.logsumexp(s, 0).item()) < 1e-12


def test_lse_merges_with_a_disjoint_token_set():
    # attention over visual + text tokens equals the lse-weighted merge of
    # the two parts: the quantity a caller combines with the text part
    p = Params(2, 4, 4, 1, 64, 2, 8)
    kr, vr = _pair(p, 3)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 64))
    kt, vt = rng.standard_normal((5, 64)), rng.standard_normal((5, 64))
    scale = 0.125
    o_v, l_v = attend(kr, vr, p, q, scale)
    s_t = scale * (kt @ q[0])
    l_t = np.log(np.sum(np.exp(s_t)))
    o_t = np.exp(s_t - l_t) @ vt
    w = np.exp(np.array([l_v[0], l_t]) - np.logaddexp(l_v[0], l_t))
    merged = w[0] * o_v[0] + w[1] * o_t
    K = decompress(kr, p, None).reshape(-1, 64)
    V = decompress(vr, p, None).reshape(-1, 64)
    s = scale * (np.vstack([K, kt]) @ q[0])
    full = np.exp(s - np.log(np.sum(np.exp(s)))) @ np.vstack([V, vt])
    np.testing.assert_allclose(merged, full, rtol=1e-12, atol=1e-13)


def test_transform_identities_of_the_fused_kernel():
    # k_t = sum_f B[t, f] c_f with B the orthonormal inverse 3-D DCT, so
    # q . k_t = IDCT3(q . c_f)[t] and sum_t p_t v_t = sum_f DCT3(p)[f] c'_f
    rng = np.random.default_rng(5)
    S, H, W, d = 4, 3, 5, 16
    c = rng.standard_normal((S, H, W, d))        # coefficients of one head
    cv = rng.standard_normal((S, H, W, d))
    q = rng.standard_normal(d)
    k = dct3_inverse(c[:, :, :, None, :])[:, :, :, 0, :]
    v = dct3_inverse(cv[:, :, :, None, :])[:, :, :, 0, :]
    s = dct3_inverse((c @ q)[..., None, None])[..., 0, 0]
    np.testing.assert_allclose(s, k @ q, rtol=1e-12, atol=1e-12)
    pr = np.exp(s - s.max())
    pr /= pr.sum()
    P = dct3_forward(pr[..., None, None])[..., 0, 0]
    np.testing.assert_allclose(np.tensordot(P, cv, axes=3),
                               np.tensordot(pr, v, axes=3), rtol=1e-12, atol=1e-12)
