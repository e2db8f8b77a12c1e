"""Parity of the HIP path with the CPU oracle, step by step and end to end.

Every test calls the library through its C ABI (the ctypes binding) on
seeded synthetic inputs and compares with the oracle on the same inputs.
The stage entry points run the kernels tact_compress and tact_decompress
launch, stopped after (or started at) one step:
  * DCT coefficients:  ||c_gpu - c_ref|| / ||c_ref|| <= 1e-5 per unit
  * variances:         given the coefficients the kernels computed, within
                       1e-6 relative per bin (fp32 sums of squares); against
                       the exact coefficients, |sqrt(v_gpu) - sqrt(v_ref)| is
                       bounded by the bin's RMS coefficient error (the
                       triangle inequality) plus that rounding
  * bits:              bit-exact given identical variances
  * records:           byte-exact given identical coefficients and
                       variances (both sides decide in fp32; the coding
                       stage codes the values as given, without rotation)
  * dequantize:        every code recovered exactly; values within the
                       decoding kernel's split-fp16 rounding (2^-19)
  * decompress:        bf16 outputs equal except where the exact value
                       lies within the transform's error bound (1e-5 of
                       the RMS) of a bf16 rounding boundary
  * end to end:        bits equal except at the cut, codes >= 99.99% equal
                       with mismatches next to a threshold (of the rotated
                       value when the rotation is on), and round-trip MSE
                       within 1e-3 relative.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from tact_inputs import WORKLOADS, generate_unit, generate_units

pytestmark = pytest.mark.gpu

if torch.cuda.device_count() > 0:
    import kv_cache_compression_tact_amd as tact


def say(*a):
    print(*a, flush=True)


def _geom(S, H, W, hk, d, budget, bmax=8, dtype=torch.bfloat16, **kw):
    return tact.Geometry(S, H, W, hk, d, budget, max_bits=bmax, dtype=dtype, **kw)


def _oparams(g):
    return O.Params(g.S, g.H, g.W, g.kv_heads, g.head_dim, g.budget_bits, g.max_bits)


def _orot(g):
    return "hadamard" if g.rotation == tact.ROTATION_HADAMARD else "none"


def _oquant(g):
    return O.QUANTIZERS[g.quantizer]


def _units(g, n, seed=0, scale_spike=True):
    """n random correlated units of geometry g (AR(1) field + spikes), on GPU."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((n,) + g.unit_shape, generator=gen, dtype=torch.float64)
    for ax, rho in ((1, 0.9), (2, 0.85), (3, 0.8)):
        for i in range(1, x.shape[ax]):
            cur = x.select(ax, i)
            cur.mul_(math.sqrt(1 - rho * rho)).add_(x.select(ax, i - 1), alpha=rho)
    if scale_spike:
        sc = torch.ones(g.kv_heads * g.head_dim, dtype=torch.float64)
        sc[torch.randperm(sc.numel(), generator=gen)[:3]] = 8.0
        x = x * sc.view(g.kv_heads, g.head_dim)
    return x.to(g.dtype).cuda()


GEOMS = [
    # (S, H, W, kv_heads, head_dim, budget, bmax, dtype)
    (4, 8, 8, 2, 64, 1, 3, torch.float32),          # the tiny workload shape
    (5, 7, 9, 3, 64, 2, 8, torch.bfloat16),         # ragged everywhere
    (3, 14, 14, 1, 128, 1, 8, torch.bfloat16),
    (2, 5, 3, 2, 256, 4, 8, torch.bfloat16),
    (33, 3, 2, 1, 128, 3, 5, torch.bfloat16),       # S beyond 32
    (64, 2, 3, 1, 64, 1, 8, torch.float32),
    # wider planes: every H / W contraction size of the plane kernels
    (3, 17, 23, 2, 128, 2, 8, torch.bfloat16),
    (2, 10, 21, 1, 64, 1, 8, torch.float32),
    (2, 20, 12, 2, 64, 3, 8, torch.bfloat16),
    (2, 26, 30, 1, 128, 1, 8, torch.bfloat16),
]


# W beyond 32: the H and W axes run as separate passes
GEOMS_AXIS_PATH = [
    (3, 5, 40, 1, 128, 2, 8, torch.bfloat16),
    (2, 36, 3, 2, 64, 1, 8, torch.float32),
]


def _gpu(a):
    """A numpy array as a contiguous GPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("geo", GEOMS + GEOMS_AXIS_PATH)
def test_dct_forward_and_inverse(geo):
    g = _geom(*geo)
    say("dct", geo)
    x = _units(g, 2, seed=1)
    c = tact.dbg_dct3(x, g).cpu().numpy()
    xs = x.float().cpu().numpy().astype(np.float64)
    for u in range(2):
        e = _rel(c[u], O.dct3_forward(xs[u]))
        say(f"  forward rel err {e:.3e}")
        assert e <= 1e-5
    y = tact.dbg_dct3(torch.from_numpy(c).cuda(), g, inverse=True).cpu().numpy()
    for u in range(2):
        e = _rel(y[u], O.dct3_inverse(c[u].astype(np.float64)))
        say(f"  inverse rel err {e:.3e}")
        assert e <= 1e-5
        # forward then inverse: two transforms, each within 1e-5
        assert _rel(y[u], xs[u]) <= 2e-5


@pytest.mark.parametrize("axes", [1, 2, 4, 3, 6, 5, 0])
def test_dct_axis_subsets(axes):
    g = _geom(5, 6, 7, 2, 64, 1, axes=axes)
    say("dct axes", axes)
    x = _units(g, 1, seed=2)
    c = tact.dbg_dct3(x, g).cpu().numpy()[0]
    ax = tuple(a for a in range(3) if axes & (1 << a))
    ref = O.dct3_forward(x.float().cpu().numpy()[0].astype(np.float64), ax)
    assert _rel(c, ref) <= 1e-5


def _check_variances(x, g, units=None):
    """Variances of the cache tensors x as the allocation reads them."""
    g0 = tact.Geometry(*g.unit_shape, budget_bits=g.budget_bits, max_bits=g.max_bits,
                       dtype=g.dtype, axes=g.axes, quantizer=g.quantizer, rotation=0)
    var = tact.dbg_bin_variance(x, g).cpu().numpy().astype(np.float64)
    c = tact.dbg_dct3(x, g0).cpu().numpy()
    axes = tuple(a for a in range(3) if g.axes & (1 << a))
    worst_red = worst_ex = 0.0
    for u in (range(x.shape[0]) if units is None else units):
        xs = x[u].float().cpu().numpy().astype(np.float64)
        r, e = _variance_bounds(var[u], c[u], O.dct3_forward(xs, axes), g.rotation)
        worst_red, worst_ex = max(worst_red, r), max(worst_ex, e)
    red = f"reduction {worst_red:.2e} relative, " if g.rotation == 0 else ""
    say(f"  variances: {red}exact-coefficient bound used to {worst_ex:.2f}")
    return var


def _variance_bounds(var, c, ref_c, rotation):
    """Variances var (..., bins) the kernels computed, against the
    coefficients c the same kernels computed (unrotated, fp32) and the exact
    ones ref_c (fp64), both (..., head_dim).  Returns the worst relative
    reduction error and the worst use of the exact-coefficient bound."""
    var = np.asarray(var, dtype=np.float64)
    ref = O.bin_variance(ref_c)
    cu = np.asarray(c, dtype=np.float64)
    pos = ref > 0
    worst_red = 0.0
    if rotation == 0:
        # the reduction alone: the same kernels' coefficients, summed in fp64
        mine = O.bin_variance(cu)
        red = np.abs(var - mine)[pos] / mine[pos]
        worst_red = float(red.max())
        assert np.all(red <= 1e-6)
    # against the exact coefficients: |(|a| - |b|)| <= |a - b| for the bin
    # vectors, over sqrt(d); the rotation (orthonormal) adds its fp32
    # rounding (six butterfly stages) to that of the sums
    dc = np.sqrt(np.mean((cu - ref_c) ** 2, axis=-1))
    slack = (1e-6 if rotation == 0 else 2e-6) * np.sqrt(ref)
    lhs = np.abs(np.sqrt(var) - np.sqrt(ref))
    assert np.all(lhs <= dc + slack)
    return worst_red, float(np.max((lhs / (dc + slack))[pos]))


@pytest.mark.parametrize("rot", [0, 1])
@pytest.mark.parametrize("geo", GEOMS + GEOMS_AXIS_PATH)
def test_bin_variance(geo, rot):
    g = _geom(*geo, rotation=rot)
    say("variance", geo, "rotation", rot)
    _check_variances(_units(g, 2, seed=8), g)


def _var_cases(rng, nb):
    v = np.exp(rng.normal(0.0, 4.0, nb)).astype(np.float32)
    out = [v.copy()]
    w = v.copy()
    w[::7] = w[0]                       # exact ties
    w[1::11] = w[1] * np.float32(4.0)   # ties across bit levels
    w[2::13] = 0.0                      # dead bins
    out.append(w)
    out.append(np.zeros(nb, np.float32))                       # all dead
    q = np.full(nb, 2.0, np.float32)                           # all equal
    out.append(q)
    sub = v.copy()
    sub[:nb // 3] = np.float32(1e-42)                          # fp32 subnormals
    out.append(sub)
    return out


@pytest.mark.parametrize("geo,budget,bmax", [
    ((4, 8, 8, 2, 64), 1, 3), ((5, 7, 9, 3, 64), 2, 8), ((3, 14, 14, 1, 128), 1, 8),
    ((1, 1, 3, 1, 64), 1, 2), ((2, 5, 3, 2, 256), 4, 8), ((7, 3, 5, 1, 64), 0, 8),
    ((7, 3, 5, 1, 64), 8, 8), ((6, 6, 6, 4, 64), 3, 4),
    # several allocation workgroups per unit (about 16K bins each): ties at the
    # cut are then shared out across slices in bin order
    ((16, 32, 32, 3, 64), 1, 8), ((32, 24, 24, 4, 128), 2, 5),
])
def test_allocation_bit_exact(geo, budget, bmax):
    g = _geom(*geo, budget, bmax)
    say("allocate", geo, budget, bmax)
    rng = np.random.default_rng(sum(geo) + budget)
    cases = _var_cases(rng, g.n_bins)
    var = torch.from_numpy(np.stack(cases).reshape((len(cases),) + g.unit_shape[:-1]))
    bits = tact.dbg_allocate(var.cuda(), g).cpu().numpy().reshape(len(cases), -1)
    for u, v in enumerate(cases):
        ref = O.allocate_bits(v.astype(np.float64), budget * g.n_bins, bmax)
        assert np.array_equal(bits[u].astype(np.int64), ref), u


@pytest.mark.parametrize("geo", [(3, 4, 5, 2, 64), (32, 24, 24, 4, 128)])
def test_uniform_allocation(geo):
    g = _geom(*geo, 3, 8, alloc_mode=tact.ALLOC_UNIFORM)
    var = torch.rand((2,) + g.unit_shape[:-1]).cuda()
    bits = tact.dbg_allocate(var, g).cpu()
    assert torch.all(bits == 3)


def _check_records_given_inputs(coef, g):
    """Records of fp32 coefficients (units on the CPU) with the allocation of
    their fp32 variances: byte-exact against the oracle's."""
    op = _oparams(g)
    var = np.stack([O.bin_variance(cu.astype(np.float64)) for cu in coef]).astype(np.float32)
    coef = coef.astype(np.float32)
    rec = tact.dbg_quantize(_gpu(coef), _gpu(var), g).cpu().numpy()
    for u in range(coef.shape[0]):
        v = var[u].astype(np.float64)
        b = O.allocate_bits(v, O.total_bits(op), g.max_bits).reshape(v.shape)
        gg = O.gains_f32(v)
        ref = O.pack_record(O.quantize(coef[u], gg, b), gg, b, op)
        assert np.array_equal(rec[u], ref), (u, int(np.sum(rec[u] != ref)))


@pytest.mark.parametrize("geo", GEOMS)
def test_quantize_pack_byte_exact(geo):
    g = _geom(*geo, rotation=0)
    say("quantize", geo)
    rng = np.random.default_rng(3)
    U = 2
    coef = (rng.standard_t(3, (U,) + g.unit_shape) *
            np.exp(rng.normal(0, 2, (U,) + g.unit_shape[:-1]))[..., None]).astype(np.float32)
    coef[0, 0, 0, 0, 0, :] = 0.0        # a zero-energy bin
    _check_records_given_inputs(coef, g)


def _check_dequantize(recs, g):
    """Decoding stage on records (CPU uint8): every code comes back exactly,
    the values within the decoding kernel's split-fp16 rounding."""
    op = _oparams(g)
    deq = tact.dbg_dequantize(_gpu(recs), g).cpu().numpy().astype(np.float64)
    worst = 0.0
    for u in range(recs.shape[0]):
        c, gg, b = O.unpack_record(recs[u], op)
        ref = O.dequantize(c, gg, b)
        err = np.abs(deq[u] - ref)
        assert np.all(err[ref == 0] == 0)
        nz = ref != 0
        worst = max(worst, float(np.max(err[nz] / np.abs(ref[nz]), initial=0.0)))
        assert np.all(err <= 2.0 ** -19 * np.abs(ref))
        g64 = gg.astype(np.float64)
        for nb in range(1, 9):
            sel = (b == nb) & (g64 > 0)
            if not sel.any():
                continue
            lv, _ = O.codebook_f32(nb)
            val = deq[u][sel] / g64[sel][:, None]
            back = np.argmin(np.abs(val[..., None] - lv.astype(np.float64)), axis=-1)
            assert np.array_equal(back, c[sel].astype(np.int64)), nb
    say(f"  dequantize: worst relative error {worst:.2e}")


@pytest.mark.parametrize("geo", GEOMS + GEOMS_AXIS_PATH)
def test_dequantize_recovers_every_code(geo):
    g = _geom(*geo, rotation=0)
    say("dequantize", geo)
    op = _oparams(g)
    x = _units(g, 2, seed=4).float().cpu().numpy().astype(np.float64)
    _check_dequantize(np.stack([O.compress(x[u], op, rotation="none") for u in range(2)]), g)


@pytest.mark.parametrize("rot", [1, 0])
@pytest.mark.parametrize("geo", GEOMS + GEOMS_AXIS_PATH)
def test_decompress_from_oracle_records(geo, rot):
    g = _geom(*geo, rotation=rot)
    say("decompress", geo, "rotation", rot)
    op = _oparams(g)
    x = _units(g, 2, seed=5).float().cpu().numpy().astype(np.float64)
    recs = np.stack([O.compress(x[u], op, rotation=_orot(g)) for u in range(2)])
    out = tact.decompress(torch.from_numpy(recs).cuda(), g).float().cpu().numpy()
    for u in range(2):
        exact = O.decompress(recs[u], op, None, rotation=_orot(g))
        if g.dtype == torch.bfloat16:
            _check_bf16_decode(out[u], exact, f"unit {u}")
        else:
            assert _rel(out[u], exact) <= 1e-5


@pytest.mark.parametrize("budget", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("geo", [(3, 20, 24, 2, 128), (2, 24, 12, 1, 64), (2, 28, 30, 1, 64)])
def test_decode_every_bin_at_one_width(geo, budget):
    # Uniform allocation gives every bin the same width, so each wave of the
    # decoder turns bit planes into codes at one width: 1, 2, 4 and 8 planes
    # (3 and 5 bits leave planes zero), on rows of 32 and 16 bins and with
    # rows staged in two passes (8 waves of up to 4 rows)
    g = _geom(*geo, budget, 8, dtype=torch.float32, alloc_mode=tact.ALLOC_UNIFORM)
    say("decode at one width", geo, budget)
    op = _oparams(g)
    x = _units(g, 1, seed=21).float().cpu().numpy().astype(np.float64)
    rec = O.compress(x[0], op, alloc="uniform", rotation=_orot(g))
    assert np.all(O.unpack_record(rec, op)[2] == budget)     # every bin at the one width
    out = tact.decompress(torch.from_numpy(rec[None]).cuda(), g).float().cpu().numpy()[0]
    exact = O.decompress(rec, op, "f32", rotation=_orot(g))
    assert _rel(out, exact) <= 1e-5


def _check_bf16_decode(out, exact, what):
    """bf16 decoder output (as float) against the exact decoded values
    (fp64): equal to their bf16 rounding except where the exact value lies
    within the transform's error bound (1e-5 of the RMS) of a rounding
    boundary, and then within half a bf16 ulp of it, up to that bound."""
    ref = O.round_to_bf16(exact)
    diff = O.bf16_bits(out) != O.bf16_bits(ref)
    rms = math.sqrt(np.mean(exact ** 2))
    tol = 1e-5 * rms                             # the transform's error bound
    # an entry may round differently only where its exact value lies within
    # the error bound of a bf16 rounding boundary: half an ulp above |ref|,
    # half an ulp below it (the smaller ulp when |ref| is a power of two)
    mag_r = np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(mag_r))
    ulp_up = np.ldexp(1.0, (e - 7).astype(int))
    ulp_dn = np.where(mag_r == np.ldexp(1.0, e.astype(int)), 0.5 * ulp_up, ulp_up)
    ax = np.abs(exact)
    dist = np.minimum(mag_r + 0.5 * ulp_up - ax, ax - (mag_r - 0.5 * ulp_dn))
    near = dist <= tol
    assert np.all(near[diff]), np.argwhere(diff & ~near)[:4]
    # and it is then a rounding-boundary case: the GPU value is within half a
    # bf16 ulp of the exact value, up to the error bound
    mag = np.maximum(np.abs(exact[diff]), np.abs(out[diff]))
    ulp = np.ldexp(1.0, (np.floor(np.log2(mag)) - 7).astype(int))
    assert np.all(np.abs(out[diff] - exact[diff]) <= 0.5 * ulp + tol)
    say(f"  {what}: bf16 mismatches {diff.mean():.2e} of entries, "
        f"near a boundary {near.mean():.2e}")


def _compare_records(rec_gpu, rec_ref, op, coef_ref, rotation="hadamard", quantizer="lloyd_max"):
    """End-to-end record comparison; returns stats."""
    c1, g1, b1 = O.unpack_record(rec_gpu, op)
    c2, g2, b2 = O.unpack_record(rec_ref, op)
    assert b1.sum() == b2.sum() == O.total_bits(op)
    # bits may differ only where the bin's marginal gain sits at the cut
    var_ref = O.bin_variance(coef_ref)
    differ = b1 != b2
    if differ.any():
        gains = np.sort(np.ldexp(np.repeat(var_ref.ravel(), op.max_bits),
                                 -2 * np.tile(np.arange(op.max_bits), var_ref.size)))[::-1]
        cut = gains[O.total_bits(op) - 1]
        for idx in zip(*np.nonzero(differ)):
            k = min(b1[idx], b2[idx])          # the contested bit
            gk = np.ldexp(var_ref[idx], -2 * int(k))
            assert abs(gk - cut) <= 1e-5 * cut, (idx, gk, cut)
    assert differ.mean() <= 1e-3
    np.testing.assert_allclose(g1, g2, rtol=1e-5)
    same = (b1 == b2) & (b1 > 0)
    if not same.any():                      # budget 0: no bin carries codes
        return differ.mean(), 0.0
    eq = c1[same] == c2[same]
    assert eq.mean() >= 0.9999
    # every mismatching code sits next to a decision threshold
    if (~eq).any():
        # the value the quantizer decides on: c / g, rotated.  The gain is
        # an input of the coding step and is checked on its own above, so
        # the oracle coefficient is scaled by the record's own gain: the
        # distance then measures the coefficient error alone
        u_all = coef_ref[same] / g1[same][:, None].astype(np.float64)
        if rotation == "hadamard":
            u_all = O.rotate(u_all)
        u = u_all[~eq]
        gm = g1[same][:, None].repeat(op.head_dim, 1)[~eq].astype(np.float64)
        bb = b1[same][:, None].repeat(op.head_dim, 1)[~eq]
        # the coefficient scale the transform's 1e-5 agreement is stated at
        sigma = float(np.sqrt(np.mean(coef_ref.astype(np.float64) ** 2)))
        worst = worst_t = 0.0
        for ui, gi, bi in zip(u, gm, bb):
            _, thr = O.codebook_f32(int(bi), quantizer)
            t = float(thr[np.argmin(np.abs(thr - ui))])
            # within 1e-5 relative of the threshold, the relative scale being
            # the larger of |t| and the unit's coefficient RMS in this bin's
            # gain units (the only scale at t = 0)
            dist = abs(ui - t) / max(abs(t), sigma / gi)
            worst = max(worst, dist)
            if t != 0.0:
                worst_t = max(worst_t, abs(ui - t) / abs(t))
            assert dist <= 1e-5, (ui, t, gi, sigma, dist)
        say(f"  {int((~eq).sum())} code mismatches, worst normalised distance {worst:.2e}"
            f" (relative to |t| alone: {worst_t:.2e})")
    return differ.mean(), 1 - eq.mean()


@pytest.mark.parametrize("rot", [1, 0])
@pytest.mark.parametrize("geo", GEOMS + GEOMS_AXIS_PATH)
def test_compress_end_to_end(geo, rot):
    g = _geom(*geo, rotation=rot)
    say("compress", geo, "rotation", rot)
    op = _oparams(g)
    x = _units(g, 2, seed=6)
    rec = tact.compress(x, g.budget_bits, g.max_bits, rotation=rot).cpu().numpy()
    xs = x.float().cpu().numpy().astype(np.float64)
    for u in range(2):
        ref = O.compress(xs[u], op, rotation=_orot(g))
        _compare_records(rec[u], ref, op, O.dct3_forward(xs[u]), _orot(g))


def _roundtrip_check(x_gpu, g, units=None):
    op = _oparams(g)
    axes = tuple(a for a in range(3) if g.axes & (1 << a))
    alloc = "uniform" if g.alloc_mode == tact.ALLOC_UNIFORM else "waterfill"
    out, rec = tact.roundtrip(x_gpu, g.budget_bits, g.max_bits, axes=g.axes,
                              alloc_mode=g.alloc_mode, rotation=g.rotation,
                              quantizer=g.quantizer)
    units = range(x_gpu.shape[0]) if units is None else units
    for u in units:
        xs = x_gpu[u].float().cpu().numpy().astype(np.float64)
        c = tact.dbg_dct3(x_gpu[u:u + 1], g).cpu().numpy()[0]
        e = _rel(c, O.dct3_forward(xs, axes))
        say(f"  unit {u}: forward rel err {e:.3e}")
        assert e <= 1e-5
        od = "bf16" if g.dtype == torch.bfloat16 else "f32"
        ref_out, ref_rec = O.roundtrip(xs, op, od, axes, alloc, _orot(g), _oquant(g))
        m_gpu = O.mse(out[u].float().cpu().numpy(), xs)
        m_ref = O.mse(ref_out, xs)
        say(f"  unit {u}: mse gpu {m_gpu:.6e} oracle {m_ref:.6e}")
        assert abs(m_gpu / m_ref - 1) <= 1e-3
        _compare_records(rec[u].cpu().numpy(), ref_rec, op, O.dct3_forward(xs, axes), _orot(g),
                         _oquant(g))


@pytest.mark.parametrize("geo", GEOMS + GEOMS_AXIS_PATH)
def test_roundtrip_small(geo):
    g = _geom(*geo)
    say("roundtrip", geo)
    _roundtrip_check(_units(g, 3, seed=7), g)


def _random_geometries(n, seed):
    # seeded shapes across every kernel size class: S, H, W from 1 (a
    # one-point DCT) to 64 / 32 / 32, 1..3 kv heads, every head_dim, any
    # budget up to the cap, both dtypes and both rotations
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        S, H, W = int(rng.integers(1, 65)), int(rng.integers(1, 33)), int(rng.integers(1, 33))
        hk, d = int(rng.integers(1, 4)), int(rng.choice([64, 128, 256]))
        if S * H * W * hk * d > 60000:
            continue
        bmax = int(rng.integers(1, 9))
        budget = int(rng.integers(0, bmax + 1))
        dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
        out.append((S, H, W, hk, d, budget, bmax, dtype, int(rng.random() < 0.8)))
    return out


@pytest.mark.parametrize("geo", _random_geometries(12, 2026))
def test_stages_random_geometries(geo):
    """Every stage entry point on the seeded random geometries: variances
    (against the same kernels' coefficients and the exact ones), bits given
    the GPU's variances, records given identical inputs (geometries whose
    coding runs in the plane pass) and the decoding stage."""
    *shape, rot = geo
    g = _geom(*shape, rotation=rot)
    g0 = _geom(*shape, rotation=0)
    say("stages random", geo)
    op = _oparams(g)
    x = _units(g, 2, seed=sum(shape[:5]) + 1)
    var = _check_variances(x, g).astype(np.float32)
    bits = tact.dbg_allocate(_gpu(var), g).cpu().numpy().reshape(2, -1)
    for u in range(2):
        ref = O.allocate_bits(var[u].astype(np.float64).ravel(), O.total_bits(op), g.max_bits)
        assert np.array_equal(bits[u].astype(np.int64), ref), u
    xs = x.float().cpu().numpy().astype(np.float64)
    coef = np.stack([O.dct3_forward(xs[u]) for u in range(2)]).astype(np.float32)
    if g.H <= 32 and g.W <= 32 and g.H * g.W * 256 <= 150 * 1024:
        _check_records_given_inputs(coef, g0)
    _check_dequantize(np.stack([O.compress(xs[u], op, rotation="none") for u in range(2)]), g0)


@pytest.mark.parametrize("geo", _random_geometries(12, 2026))
def test_roundtrip_random_geometries(geo):
    *shape, rot = geo
    g = _geom(*shape, rotation=rot)
    say("roundtrip random", geo)
    _roundtrip_check(_units(g, 2, seed=sum(shape[:5])), g)


@pytest.mark.parametrize("geo", [GEOMS[1], GEOMS[3], GEOMS_AXIS_PATH[0]])
def test_roundtrip_without_rotation(geo):
    # the rotation ablation: the normalized coefficients quantized as they are
    g = _geom(*geo, rotation=0)
    say("roundtrip no rotation", geo)
    _roundtrip_check(_units(g, 2, seed=13), g)


@pytest.mark.parametrize("quant", [1, 2])
@pytest.mark.parametrize("rot", [1, 0])
@pytest.mark.parametrize("geo", [GEOMS[1], GEOMS[3], GEOMS[6], GEOMS_AXIS_PATH[0]])
def test_roundtrip_quantizer_backends(geo, rot, quant):
    # the page's quantizer comparison: symmetric uniform and NormalFloat
    # tables with absmax gains (records, gains and round-trip MSE)
    g = _geom(*geo, rotation=rot, quantizer=quant)
    say("roundtrip quantizer", quant, geo, "rotation", rot)
    _roundtrip_check(_units(g, 2, seed=15), g)


@pytest.mark.parametrize("quant", [1, 2])
def test_decompress_quantizer_backends_from_oracle_records(quant):
    g = _geom(3, 17, 23, 2, 128, 2, 8, torch.float32, quantizer=quant)
    op = _oparams(g)
    xs = _units(g, 2, seed=16).cpu().numpy().astype(np.float64)
    recs = np.stack([O.compress(xs[u], op, quantizer=_oquant(g)) for u in range(2)])
    out = tact.decompress(torch.from_numpy(recs).cuda(), g).cpu().numpy()
    for u in range(2):
        ref = O.decompress(recs[u], op, None, quantizer=_oquant(g))
        e = _rel(out[u], ref)
        say(f"  quantizer {quant} unit {u}: rel err {e:.2e}")
        assert e <= 1e-5


def test_rotation_spreads_a_spike_channel():
    # one channel x64 louder than the rest: at 8 bits the identity clips it,
    # the rotation spreads it over the 64 coordinates of its word
    g = _geom(4, 8, 8, 2, 64, 8, 8, dtype=torch.float32)
    x = _units(g, 1, seed=14, scale_spike=False)
    x[..., 0, 5] *= 64.0
    e = {}
    for rot in (0, 1):
        out, _ = tact.roundtrip(x, 8, 8, rotation=rot)
        e[rot] = O.mse(out[0].cpu().numpy(), x[0].cpu().numpy())
    say("spike mse", e)
    assert e[1] < 0.1 * e[0]


@pytest.mark.parametrize("axes", [1, 2, 4, 3, 5, 6, 0])
def test_roundtrip_axis_subsets(axes):
    # the page's transform ablation: 1- and 2-axis DCTs, and no transform
    # (axes 0), through the codec
    g = _geom(5, 7, 9, 2, 64, 2, axes=axes)
    say("roundtrip axes", axes)
    _roundtrip_check(_units(g, 2, seed=11), g)


@pytest.mark.parametrize("geo", [(4, 8, 8, 2, 64, 1, 3, torch.float32), (3, 14, 14, 1, 128, 2, 8, torch.bfloat16)])
def test_roundtrip_uniform_allocation(geo):
    # the page's allocation ablation: every bin at the average budget
    g = _geom(*geo, alloc_mode=tact.ALLOC_UNIFORM)
    say("roundtrip uniform", geo)
    _roundtrip_check(_units(g, 2, seed=12), g)


def test_tiny_workload_all_units():
    wl = WORKLOADS["tiny"]
    say("tiny workload")
    x = generate_units(wl, device="cuda")
    g = tact.Geometry(*wl.unit_shape, budget_bits=1, max_bits=3, dtype=torch.float32)
    _roundtrip_check(x, g)


def test_in_place_roundtrip_and_separate_calls_agree():
    g = _geom(5, 7, 9, 3, 64, 2)
    x = _units(g, 3, seed=8)
    out1, rec1 = tact.roundtrip(x, 2)
    rec2 = tact.compress(x, 2)
    out2 = tact.decompress(rec2, g)
    assert torch.equal(rec1, rec2) and torch.equal(out1, out2)
    y = x.clone()
    tact.roundtrip(y, 2, out=y, keep_records=False)
    assert torch.equal(y, out1)


def test_deterministic():
    g = _geom(6, 6, 6, 4, 64, 2)
    x = _units(g, 4, seed=9)
    a = tact.compress(x, 2)
    b = tact.compress(x, 2)
    assert torch.equal(a, b)


def test_strided_units_and_empty_batch():
    g = _geom(3, 5, 4, 2, 64, 1)
    big = _units(g, 4, seed=10)
    view = big[::2]                          # unit stride = 2 units
    rec = tact.compress(view, 1)
    ref = tact.compress(view.contiguous(), 1)
    assert torch.equal(rec, ref)
    empty = big[:0]
    assert tact.compress(empty, 1).shape[0] == 0


def test_batched_units_match_single_unit_calls():
    """A unit's result does not depend on the batch around it: a full ct4b
    launch (68 units, memory system under load) against single-unit calls,
    bit for bit, for the transform and for the whole codec."""
    wl = WORKLOADS["ct4b"]
    say("batched vs single, ct4b units", wl.n_units)
    x = generate_units(wl, device="cuda")
    g = tact.Geometry(*wl.unit_shape, budget_bits=1, max_bits=wl.max_bits, dtype=wl.dtype)
    c_all = tact.dbg_dct3(x, g)
    out_all, rec_all = tact.roundtrip(x, 1, wl.max_bits)
    for u in (0, 33, wl.n_units - 1):
        assert torch.equal(c_all[u], tact.dbg_dct3(x[u:u + 1], g)[0]), u
        out_u, rec_u = tact.roundtrip(x[u:u + 1].contiguous(), 1, wl.max_bits)
        assert torch.equal(rec_all[u], rec_u[0]), u
        assert torch.equal(out_all[u], out_u[0]), u
    del x, c_all, out_all, rec_all
    torch.cuda.empty_cache()


FULL = [("ct4b", 1), ("ct4b", 2), ("ct4b", 4), ("ct7b", 1), ("ct32b", 1), ("video", 1), ("video", 2)]


@pytest.mark.parametrize("name,budget", FULL)
def test_full_size_sampled_units(name, budget):
    """Whole launch at the workload's full size (as the benchmark runs it);
    the first and last unit are checked against the oracle."""
    wl = WORKLOADS[name]
    say("full size", name, budget, "units", wl.n_units)
    x = generate_units(wl, device="cuda")
    g = tact.Geometry(*wl.unit_shape, budget_bits=budget, max_bits=wl.max_bits, dtype=wl.dtype)
    _roundtrip_check(x, g, units=[0, wl.n_units - 1])
    del x
    torch.cuda.empty_cache()


def test_full_size_stages_one_ct32b_unit():
    """Every stage at the full ct32b unit shape (64 x 24 x 24, 8 kv heads of
    128): coefficients, variances, bits given those variances, records given
    identical coefficients and variances, and the decoding stage."""
    wl = WORKLOADS["ct32b"]
    say("full-size stages, ct32b unit (0, 0, K)")
    x = generate_units(wl, units=[(0, 0, 0)], device="cuda")
    g = tact.Geometry(*wl.unit_shape, budget_bits=1, max_bits=wl.max_bits, dtype=wl.dtype)
    g0 = tact.Geometry(*wl.unit_shape, budget_bits=1, max_bits=wl.max_bits, dtype=wl.dtype,
                       rotation=0)
    op = _oparams(g)
    xs = x[0].float().cpu().numpy().astype(np.float64)
    ref_c = O.dct3_forward(xs)
    e = _rel(tact.dbg_dct3(x, g0).cpu().numpy()[0], ref_c)
    say(f"  forward rel err {e:.3e}")
    assert e <= 1e-5
    var = _check_variances(x, g)[0].astype(np.float32)
    bits = tact.dbg_allocate(_gpu(var[None]), g).cpu().numpy()[0]
    ref_bits = O.allocate_bits(var.astype(np.float64), O.total_bits(op), g.max_bits)
    assert np.array_equal(bits.ravel().astype(np.int64), ref_bits)
    _check_records_given_inputs(ref_c.astype(np.float32)[None], g0)
    _check_dequantize(O.compress(xs, op, rotation="none")[None], g0)
    del x
    torch.cuda.empty_cache()


# ---- units at the size cap --------------------------------------------------
# A unit's fp32 volume, with each grid axis rounded up to the 16, 32 or 64
# rows of its matrix tile, may be at most 2^30 bytes; the kernels' largest
# buffer offsets (padded rows included) occur at that cap.
CAP_GEOMS = [
    (2, 64, 64, 64, 64, 1, 8, torch.bfloat16),    # S pads 2 -> 16; H, W > 32: axis passes
    (40, 20, 18, 32, 128, 2, 8, torch.bfloat16),  # ragged on every axis; the plane pass
]


@pytest.mark.parametrize("geo", CAP_GEOMS)
def test_padded_units_at_the_size_cap(geo):
    """A unit whose padded fp32 volume is exactly 2^30 bytes, against the
    whole-unit oracle: coefficients, records and MSE of the round trip, and
    the decoder on the oracle's records."""
    g = _geom(*geo)
    say("size cap", geo)
    x = _units(g, 1, seed=31)
    _roundtrip_check(x, g)
    op = _oparams(g)
    xs = x[0].float().cpu().numpy().astype(np.float64)
    del x
    rec = O.compress(xs, op, rotation=_orot(g))
    out = tact.decompress(_gpu(rec[None]), g)[0].float().cpu().numpy()
    _check_bf16_decode(out, O.decompress(rec, op, None, rotation=_orot(g)), "decoder")
    torch.cuda.empty_cache()


# The largest units: 2^28 entries, padded volume 2^30 bytes (no padding).
# The oracle checks them where it works channel by channel (the transform
# acts on each channel alone) or head by head (the variances): sampled
# channels of the coefficients, codes, dequantized values and decoded
# output, one whole head of variances, and every bin's bits and gain.
LARGEST = [
    (64, 32, 32, 32, 128),   # the fused layout: the S pass, then the H/W plane pass
    (64, 64, 64, 16, 64),    # H and W beyond 32: three axis passes
]


def _correlated_unit_on_gpu(g, seed):
    """One correlated unit (AR(1) along S, H and W), drawn on the GPU."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn((1,) + g.unit_shape, generator=gen, device="cuda")
    for ax, rho in ((1, 0.9), (2, 0.85), (3, 0.8)):
        for i in range(1, x.shape[ax]):
            x.select(ax, i).mul_(math.sqrt(1 - rho * rho)).add_(x.select(ax, i - 1), alpha=rho)
    return x.to(g.dtype)


@pytest.mark.parametrize("shape", LARGEST)
def test_largest_units_sampled(shape):
    kv, d = shape[3], shape[4]
    g = tact.Geometry(*shape, budget_bits=1, max_bits=8, dtype=torch.bfloat16, rotation=0)
    op = _oparams(g)
    fused = shape[1] <= 32 and shape[2] <= 32
    say("largest unit", shape, "fused" if fused else "axis passes")
    x = _correlated_unit_on_gpu(g, 41)
    chans = [(0, 0), (kv - 1, d - 1), (kv // 2, 63), (1, d // 2 + 1)]
    ks = torch.tensor([k for k, _ in chans], device="cuda")
    js = torch.tensor([j for _, j in chans], device="cuda")

    def pick(t):
        """(1, S, H, W, kv, d) on the GPU -> the sampled channels (S, H, W, n), fp64."""
        return t[0][..., ks, js].double().cpu().numpy()

    xs = pick(x)
    c = tact.dbg_dct3(x, g)
    cs = pick(c)
    for i, ch in enumerate(chans):
        e = _rel(cs[..., i], O.dct3_forward(xs[..., i]))
        assert e <= 1e-5, (ch, e)
    # the variances of one whole head
    hk = kv - 1
    c_head = c[0, ..., hk, :].double().cpu().numpy()
    del c
    var = tact.dbg_bin_variance(x, g)
    ref_head = O.dct3_forward(x[0, ..., hk, :].double().cpu().numpy())
    red, ex = _variance_bounds(var[0, ..., hk].cpu().numpy(), c_head, ref_head, 0)
    say(f"  head {hk}: variance reduction {red:.2e}, exact bound used to {ex:.2f}")
    # every bin's bits (from those variances) and gain, in the codec's record
    v = var[0].double().cpu().numpy()
    bits_ref = O.allocate_bits(v, O.total_bits(op), g.max_bits).reshape(v.shape)
    assert np.array_equal(tact.dbg_allocate(var, g)[0].cpu().numpy(), bits_ref)
    out, rec = tact.roundtrip(x, 1, 8, rotation=0)
    del x
    lay = O.record_layout(op)
    r0 = rec[0].cpu().numpy()
    bits = r0[lay["bits"]:lay["bits"] + op.n_bins].reshape(v.shape)
    gains = r0[lay["gains"]:lay["gains"] + 4 * op.n_bins].view("<f4").reshape(v.shape)
    assert np.array_equal(bits, bits_ref)
    assert np.array_equal(gains, O.gains_f32(v))
    # the sampled channels' codes (read back through the decoding stage),
    # their values and the decoded output
    deq = pick(tact.dbg_dequantize(rec, g))
    outs = pick(out)
    del out, rec
    sigma = float(np.sqrt(np.mean(cs ** 2)))
    for i, (k, j) in enumerate(chans):
        b, gk = bits[..., k], gains[..., k]
        g64 = gk.astype(np.float64)
        codes = np.zeros(b.shape, dtype=np.uint8)
        for nb in range(1, 9):
            sel = (b == nb) & (g64 > 0)
            if sel.any():
                lv, _ = O.codebook_f32(nb)
                val = deq[..., i][sel] / g64[sel]
                codes[sel] = np.argmin(np.abs(val[:, None] - lv.astype(np.float64)), axis=-1)
        exact = O.dequantize(codes[..., None], gk, b)[..., 0]
        assert np.all(np.abs(deq[..., i] - exact) <= 2.0 ** -19 * np.abs(exact))
        ref_codes = O.quantize(cs[..., i:i + 1], gk, b)[..., 0]
        miss = (codes != ref_codes) & (b > 0)
        if fused:
            # the coding pass reads the very coefficients the stage call returned
            assert not miss.any(), int(miss.sum())
        else:
            # the coding epilogue recomputes the last axis: a code may differ
            # only next to a threshold (the end-to-end rule)
            for idx in zip(*np.nonzero(miss)):
                _, thr = O.codebook_f32(int(b[idx]))
                u = float(np.float32(cs[idx + (i,)]) * (np.float32(1) / gk[idx]))
                t = float(thr[np.argmin(np.abs(thr - u))])
                assert abs(u - t) <= 1e-5 * max(abs(t), sigma / float(gk[idx])), (idx, u, t)
        _check_bf16_decode(outs[..., i], O.dct3_inverse(exact), f"channel ({k}, {j})")
    torch.cuda.empty_cache()


def test_small_workspace_splits_the_batch_into_chunks():
    """A workspace that holds two units splits a five-unit batch into three
    chunks; records and decoded caches equal the one-chunk call bit for bit
    (compress, decompress and the round trip, in place too)."""
    g = _geom(5, 7, 9, 3, 64, 2)
    x = _units(g, 5, seed=21)
    ws_all = tact.workspace(g, 5)
    ws_two = tact.workspace(g, 2)
    assert ws_two.numel() < ws_all.numel()
    say("chunked: workspace", ws_two.numel(), "of", ws_all.numel())
    rec1 = tact.compress(x, 2, ws=ws_all)
    rec3 = tact.compress(x, 2, ws=ws_two)
    assert torch.equal(rec1, rec3)
    out1 = tact.decompress(rec1, g, ws=ws_all)
    out3 = tact.decompress(rec1, g, ws=ws_two)
    assert torch.equal(out1, out3)
    rt_out, rt_rec = tact.roundtrip(x, 2, ws=ws_two)
    assert torch.equal(rt_rec, rec1) and torch.equal(rt_out, out1)
    y = x.clone()
    tact.roundtrip(y, 2, out=y, keep_records=False, ws=ws_two)
    assert torch.equal(y, out1)
