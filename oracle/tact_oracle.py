"""Plain CPU fp64 oracle of the TACT-KV visual-KV-cache codec.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: it exists so that tests, the smoke check and the CPU
baseline leg of the benchmark can check the HIP library against an
independent, slow, obviously correct implementation.  It shares no code,
tables or constants with the library under ``kv_cache_compression_tact_amd``.

Source of the method.  Everything below follows the AI-summary page
"TACT-KV: Tri-Axis Cosine Transform for Compressing Volumetric KV Caches in
Medical VLMs" (ai.info), mainly its section "Methodology in Plain English"
(stages 1-4 and the decoding paragraph after them), "Key Contributions"
items 1-3 and the authors' abstract at the bottom of that page.  Citations in
the docstrings use these short forms:

  [Method/1..4]   "Methodology in Plain English", numbered stage 1..4
  [Method/dec]    the decoding paragraph that follows stage 4
  [Contrib/k]     "Key Contributions", item k
  [Findings/SQ]   "Main Findings", bullet on gain-shape scalar quantization
  [Findings/batch] "Main Findings", bullet on batch and throughput at equal HBM
  [Abstract]      "Authors' abstract"

Where the page leaves a step open, the plain reading taken here is stated in
the docstring as READING; the same readings are listed in the design notes.

Precision.  All arithmetic is float64 except the one place where floating
point decides an integer that the GPU also decides: the quantization cell
index (``quantize``) is decided in float32, in the same operations and order
as the kernel (gain = sqrt(variance) rounded to fp32, r = 1/gain in fp32,
u = coefficient * r in fp32, cell = number of fp32 thresholds <= u).

Pins.  Every function here is pinned by CPU tests to facts other than its
own code: scipy's orthonormal DCT, Parseval, exact inversion, the reverse
water-filling closed form, Theorem 1's ratio on the continuous model,
brute-force integer allocation, Lloyd-Max optimality conditions and the
textbook Gaussian quantizer values, and a hand-derived record fixture.
The end-to-end behaviour on real caches is "parity unpinned": the pages
print no worked example of reconstructed values.
"""

from __future__ import annotations

import heapq
import math
from dataclasses import dataclass

import numpy as np
from scipy.special import erfc, ndtri

__all__ = [
    "Params", "dct2_matrix", "dct3_forward", "dct3_inverse", "bin_variance",
    "total_bits", "waterfill_theta", "waterfill_rates", "round_bits",
    "greedy_correct", "allocate_bits", "allocate_bits_by_sorting", "allocate_uniform",
    "lloyd_max", "codebook_f32", "gains_f32", "quantize", "dequantize",
    "QUANTIZERS", "uniform_levels", "nf_levels", "codebook", "gains_absmax_f32",
    "splitmix64", "rotation_signs", "rotate", "unrotate", "ROTATION_SEED",
    "record_layout", "pack_record", "unpack_record", "round_to_bf16",
    "bf16_bits", "compress", "decompress", "roundtrip", "mse",
    "spectral_flatness", "occupancy_bits", "absmax_to_std", "capacity_model", "attend",
]


# --------------------------------------------------------------------------
# Unit geometry
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Params:
    """Geometry and budget of one unit (one layer, one sequence, K or V).

    [Method/1]: the visual span of the cache is viewed as a grid with the
    slice/height/width shape inherited from the vision encoder; the trailing
    axes are the KV heads and the head feature dimension.
    READING: the unit tensor is (S, H, W, kv_heads, head_dim), row-major.
    [Method/3]: a per-layer bit budget; READING: ``budget_bits`` is the
    average number of code bits per entry, so the pool of T = budget_bits *
    n_bins bit-planes is shared by all heads of the unit; each bit-plane of a
    bin costs head_dim bits.  ``max_bits`` is the per-bin cap (8 on the page).
    """
    S: int
    H: int
    W: int
    kv_heads: int
    head_dim: int
    budget_bits: int
    max_bits: int = 8

    @property
    def n_bins(self) -> int:
        return self.S * self.H * self.W * self.kv_heads

    @property
    def n_entries(self) -> int:
        return self.n_bins * self.head_dim

    @property
    def shape(self):
        return (self.S, self.H, self.W, self.kv_heads, self.head_dim)


# --------------------------------------------------------------------------
# O1-O2: separable orthonormal 3-D DCT-II            [Method/2], [Contrib/1]
# --------------------------------------------------------------------------
def dct2_matrix(n: int) -> np.ndarray:
    """Orthonormal DCT-II matrix C (n x n), C[k, i] = a_k cos(pi (2i+1) k / 2n).

    a_0 = sqrt(1/n), a_k = sqrt(2/n) for k >= 1; C @ C.T = I, so the
    transform is lossless by itself [Method/2].
    """
    k = np.arange(n, dtype=np.float64)[:, None]
    i = np.arange(n, dtype=np.float64)[None, :]
    c = np.cos(np.pi * (2.0 * i + 1.0) * k / (2.0 * n))
    c[0, :] *= math.sqrt(1.0 / n)
    c[1:, :] *= math.sqrt(2.0 / n)
    return c


def _apply_along(mat: np.ndarray, x: np.ndarray, axis: int) -> np.ndarray:
    """y[..., k, ...] = sum_i mat[k, i] x[..., i, ...] along ``axis``."""
    y = np.tensordot(mat, x, axes=([1], [axis]))
    return np.moveaxis(y, 0, axis)


def dct3_forward(x: np.ndarray, axes=(0, 1, 2)) -> np.ndarray:
    """Forward separable DCT-II along slice, height and width [Method/2].

    x has shape (S, H, W, kv_heads, head_dim); the two feature axes are left
    untransformed.  ``axes`` selects a subset of the three grid axes (the
    page's transform ablation, "Main Findings"); the method uses all three.
    """
    y = np.asarray(x, dtype=np.float64)
    for ax in axes:
        y = _apply_along(dct2_matrix(y.shape[ax]), y, ax)
    return y


def dct3_inverse(c: np.ndarray, axes=(0, 1, 2)) -> np.ndarray:
    """Inverse of ``dct3_forward``: apply C^T along each transformed axis."""
    y = np.asarray(c, dtype=np.float64)
    for ax in axes:
        y = _apply_along(dct2_matrix(y.shape[ax]).T, y, ax)
    return y


# --------------------------------------------------------------------------
# O3: per-bin variance                               [Method/3], [Contrib/3]
# --------------------------------------------------------------------------
def bin_variance(coef: np.ndarray) -> np.ndarray:
    """Per-frequency-bin variance, estimated on the fly from the unit itself.

    A bin is one (ks, kh, kw, head) frequency of one head; its variance is
    taken over the head_dim coordinates.  READING: the second moment
    (1/d) sum_j c_j^2 with no mean removed, because the quantizer factors out
    only a norm (32 side bits per surviving bin, [Method/4]).
    Returns shape (S, H, W, kv_heads).
    """
    c = np.asarray(coef, dtype=np.float64)
    return np.mean(c * c, axis=-1)


# --------------------------------------------------------------------------
# O4-O7: reverse water-filling with integer rounding and greedy +-1 fix-up
#                                                    [Method/3], [Contrib/2]
# --------------------------------------------------------------------------
def total_bits(p: Params) -> int:
    """T: the number of bit-planes the unit may spend (budget * bins)."""
    if not (0 <= p.budget_bits <= p.max_bits):
        raise ValueError("budget must lie in [0, max_bits]")
    return p.budget_bits * p.n_bins


def waterfill_rates(var: np.ndarray, theta: float, bmax: int) -> np.ndarray:
    """Continuous reverse water-filling rates R_i = clamp(log2(s_i^2/theta)/2, 0, bmax).

    Bins whose variance is below the water level theta get rate 0 (their
    distortion is their variance); the others get distortion theta.
    """
    v = np.asarray(var, dtype=np.float64).ravel()
    r = np.zeros_like(v)
    pos = v > 0
    r[pos] = 0.5 * np.log2(v[pos] / theta)
    return np.clip(r, 0.0, float(bmax))


def waterfill_theta(var: np.ndarray, total: int, bmax: int,
                    iters: int = 400) -> float:
    """Water level theta with sum_i R_i(theta) = total, found by bisection.

    Bisection on log(theta) over [min positive variance * 4^-bmax,
    max variance], in float64, until the bracket ratio is below 1 + 2^-50
    or ``iters`` halvings.  Returns nan when no bin has positive variance.
    """
    v = np.asarray(var, dtype=np.float64).ravel()
    pos = v[v > 0]
    if pos.size == 0:
        return float("nan")
    lo = float(pos.min()) * 4.0 ** (-bmax)   # every positive bin at bmax
    hi = float(pos.max())                     # every bin at 0
    if total <= 0:
        return hi
    if total >= bmax * pos.size:
        return lo
    for _ in range(iters):
        mid = math.sqrt(lo * hi)
        if not (lo < mid < hi) or hi / lo < 1.0 + 2.0 ** -50:
            break
        if waterfill_rates(v, mid, bmax).sum() >= total:
            lo = mid     # still spends at least the budget: raise the level
        else:
            hi = mid
    return lo


def round_bits(var: np.ndarray, theta: float, bmax: int) -> np.ndarray:
    """Integer rounding of the continuous rates without logarithms.

    b_i = min(bmax, #{k >= 1 : s_i^2 >= theta * 2^(2k-1)}), which is
    round-half-up of R_i(theta); every product is theta times a power of two,
    so each comparison is exact in float64.
    """
    v = np.asarray(var, dtype=np.float64).ravel()
    b = np.zeros(v.shape, dtype=np.int64)
    if not math.isfinite(theta):
        return b
    for k in range(1, bmax + 1):
        b += (v >= math.ldexp(theta, 2 * k - 1)).astype(np.int64)
    return b


def _gain_key(v: float, b: int) -> float:
    """Marginal distortion of the (b+1)-th bit of a bin: s^2 * 4^-b, exact."""
    return math.ldexp(float(v), -2 * int(b))


def greedy_correct(var: np.ndarray, bits: np.ndarray, total: int,
                   bmax: int) -> np.ndarray:
    """Greedy +-1 correction until the bits sum to exactly ``total``.

    While short of the budget, give one bit to the bin whose next bit has the
    largest marginal gain s^2 4^-b (ties: smallest flat bin index).  While
    over it, take one bit from the bin whose last bit has the smallest gain
    s^2 4^-(b-1) (ties: largest flat bin index).  READING: the page names a
    +-1 greedy correction after the bisection without a tie order; this is
    the fixed order chosen.
    """
    v = np.asarray(var, dtype=np.float64).ravel()
    b = np.asarray(bits, dtype=np.int64).ravel().copy()
    s = int(b.sum())
    if s < total:
        heap = [(-_gain_key(v[i], b[i]), i) for i in range(v.size) if b[i] < bmax]
        heapq.heapify(heap)
        while s < total:
            _, i = heapq.heappop(heap)
            b[i] += 1
            s += 1
            if b[i] < bmax:
                heapq.heappush(heap, (-_gain_key(v[i], b[i]), i))
    elif s > total:
        heap = [(_gain_key(v[i], b[i] - 1), -i) for i in range(v.size) if b[i] > 0]
        heapq.heapify(heap)
        while s > total:
            _, ni = heapq.heappop(heap)
            i = -ni
            b[i] -= 1
            s -= 1
            if b[i] > 0:
                heapq.heappush(heap, (_gain_key(v[i], b[i] - 1), -i))
    return b


def allocate_bits(var: np.ndarray, total: int, bmax: int) -> np.ndarray:
    """Integer bit allocation by reverse water-filling [Method/3].

    Steps in the page's order: bisection for the water level, integer
    rounding, then the +-1 greedy correction so that the bits sum to exactly
    ``total``; capped at ``bmax``.  Returns int64 bits, flat bin order
    (ks, kh, kw, head), head fastest.
    """
    v = np.asarray(var, dtype=np.float64).ravel()
    if total <= 0:
        return np.zeros(v.shape, dtype=np.int64)
    theta = waterfill_theta(v, total, bmax)
    b = round_bits(v, theta, bmax)
    return greedy_correct(v, b, total, bmax)


def allocate_bits_by_sorting(var: np.ndarray, total: int,
                             bmax: int) -> np.ndarray:
    """Cross-check form of ``allocate_bits``: keep the ``total`` best bits.

    Lists every candidate bit (bin i, k-th bit) with its marginal gain
    s_i^2 4^-(k-1), sorts by (gain descending, bin ascending, k ascending)
    and gives each bin the number of its candidates in the first ``total``.
    Because each bin's gains decrease with k, this is the same allocation
    the greedy reaches from any threshold rounding.
    """
    v = np.asarray(var, dtype=np.float64).ravel()
    n = v.size
    if total <= 0:
        return np.zeros(n, dtype=np.int64)
    i = np.repeat(np.arange(n), bmax)
    k = np.tile(np.arange(1, bmax + 1), n)
    gain = np.ldexp(v[i], -2 * (k - 1))
    order = np.lexsort((k, i, -gain))     # last key is the primary key
    chosen = order[:total]
    return np.bincount(i[chosen], minlength=n).astype(np.int64)


# --------------------------------------------------------------------------
# O8: Lloyd-Max codebooks for a unit Gaussian         [Method/4]
# --------------------------------------------------------------------------
_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x)
    out[fin] = np.exp(-0.5 * x[fin] * x[fin]) * _INV_SQRT_2PI
    return out


def _upper_tail(x):
    """P(X > x) for X ~ N(0, 1), accurate in the upper tail."""
    return 0.5 * erfc(np.asarray(x, dtype=np.float64) / _SQRT2)


_LM_CACHE: dict = {}


def lloyd_max(bits: int):
    """MSE-optimal scalar quantizer of N(0, 1) with 2^bits cells.

    READING: the page's "precomputed Lloyd-Max table" is the Gaussian
    Lloyd-Max quantizer applied to coefficients divided by the bin gain.
    Computed on the positive half (the quantizer is symmetric; zero is a
    threshold): Lloyd iteration (thresholds at midpoints, levels at cell
    centroids E[X | cell] = (phi(a) - phi(b)) / (Q(a) - Q(b))), then Newton
    steps on the same two conditions until they hold to ~1e-15.

    Returns (levels[2^b] ascending, thresholds[2^b - 1] ascending, mse).
    Code c means the c-th level from the most negative one.
    """
    if bits in _LM_CACHE:
        return _LM_CACHE[bits]
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    m = 2 ** (bits - 1)                       # positive levels
    y = (np.arange(m) + 0.5) * (4.0 / m)      # any increasing start works

    def centroids(yv):
        t = np.concatenate([[0.0], 0.5 * (yv[:-1] + yv[1:]), [np.inf]])
        a, b = t[:-1], t[1:]
        den = _upper_tail(a) - _upper_tail(b)
        return (_phi(a) - _phi(b)) / den, t, a, b, den

    for _ in range(2000):                     # plain Lloyd iteration
        y = centroids(y)[0]
    for _ in range(60):                       # Newton on g(y) - y = 0
        g, t, a, b, den = centroids(y)
        f = g - y
        if np.max(np.abs(f)) < 1e-15:
            break
        # d centroid / d lower edge and d upper edge of each cell
        dga = _phi(a) * (g - a) / den
        fin = np.isfinite(b)
        dgb = np.zeros_like(g)
        dgb[fin] = _phi(b[fin]) * (b[fin] - g[fin]) / den[fin]
        jac = -np.eye(m)
        for j in range(m):
            # lower edge of cell j is (y[j-1] + y[j]) / 2 (or 0 for j = 0)
            if j > 0:
                jac[j, j - 1] += 0.5 * dga[j]
                jac[j, j] += 0.5 * dga[j]
            if j < m - 1:
                jac[j, j] += 0.5 * dgb[j]
                jac[j, j + 1] += 0.5 * dgb[j]
        y = y - np.linalg.solve(jac, f)
    g, t, a, b, den = centroids(y)
    levels = np.concatenate([-y[::-1], y])
    thr_pos = t[1:-1]
    thresholds = np.concatenate([-thr_pos[::-1], [0.0], thr_pos])
    # distortion: E[(X - Q(X))^2] = 1 - sum_j P(cell j) * y_j^2 (centroids)
    mse = 1.0 - 2.0 * float(np.sum(den * y * y))
    _LM_CACHE[bits] = (levels, thresholds, mse)
    return _LM_CACHE[bits]


# The scalar quantizers compared in [Findings/SQ]: the gain-shape Lloyd-Max
# table of the method, a symmetric uniform quantizer and NormalFloat.
QUANTIZERS = ("lloyd_max", "uniform", "nf")


def uniform_levels(bits: int) -> np.ndarray:
    """Symmetric uniform quantizer of [-1, 1] with 2^bits cells.

    READING: [Findings/SQ] names the backend without its construction; the
    plain one is 2^b equal cells tiling [-1, 1] with the level at each cell
    centre (mid-rise: no level at 0, so 1 bit is +-1/2), the values scaled by
    the bin's absolute maximum.
    """
    n = 2 ** bits
    return (2.0 * np.arange(n) + 1.0 - n) / n


def nf_levels(bits: int) -> np.ndarray:
    """NormalFloat levels: standard normal quantiles at the centres of 2^b
    equal-probability slices, (k + 1/2) / 2^b, normalized so that the
    outermost levels are +-1.

    READING: [Findings/SQ] names NormalFloat without its construction; this
    is the symmetric form (equal-probability quantiles, absmax scaling).
    """
    n = 2 ** bits
    # the quantiles at (k + 1/2) / 2^b mirror about 1/2: the upper half,
    # mirrored, keeps the table exactly symmetric (the middle threshold 0)
    up = ndtri((np.arange(n // 2, n) + 0.5) / n)
    up = up / up[-1]
    return np.concatenate([-up[::-1], up])


def codebook(bits: int, kind: str = "lloyd_max"):
    """(levels, thresholds) of a quantizer, ascending, float64; thresholds
    are the midpoints of adjacent levels for every kind."""
    if kind == "lloyd_max":
        levels, thresholds, _ = lloyd_max(bits)
        return levels, thresholds
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    levels = uniform_levels(bits) if kind == "uniform" else nf_levels(bits)
    if kind not in QUANTIZERS:
        raise ValueError(f"unknown quantizer {kind}")
    return levels, 0.5 * (levels[:-1] + levels[1:])


def codebook_f32(bits: int, kind: str = "lloyd_max"):
    """The table rounded to float32, as the kernel uses it."""
    levels, thresholds = codebook(bits, kind)
    return levels.astype(np.float32), thresholds.astype(np.float32)


# --------------------------------------------------------------------------
# O8b: the fixed shared orthogonal rotation            [Method/4]
# --------------------------------------------------------------------------
ROTATION_SEED = 0x54414354          # fixed: the rotation is shared by all bins
_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """SplitMix64 output for counter value x (Steele, Lea and Flood, 2014):
    z = x + 0x9E3779B97F4A7C15; z = (z ^ z>>30) * 0xBF58476D1CE4E5B9;
    z = (z ^ z>>27) * 0x94D049BB133111EB; return z ^ z>>31 (mod 2^64)."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def rotation_signs() -> np.ndarray:
    """The 64 signs s_j = +1 or -1: the top bit of SplitMix64(seed + j)."""
    return np.array([1.0 - 2.0 * (splitmix64(ROTATION_SEED + j) >> 63) for j in range(64)])


def _hadamard64() -> np.ndarray:
    from scipy.linalg import hadamard
    return hadamard(64).astype(np.float64)


def rotate(u: np.ndarray) -> np.ndarray:
    """v = R u with R = I_(d/64) (x) H_64 diag(s) / 8: the same randomized
    Hadamard rotation on every 64-coordinate block of the last axis.

    READING: the page names a fixed shared orthogonal rotation of the
    gain-normalized bin vector without giving it; this is a randomized
    Hadamard rotation in blocks of 64 coordinates (one code word), with
    Sylvester's H_64 and signs from SplitMix64.  R is orthogonal.
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    h = _hadamard64() / 8.0
    blocks = (u.reshape(u.shape[:-1] + (d // 64, 64)) * rotation_signs())
    return np.einsum("ij,...bj->...bi", h, blocks).reshape(u.shape)


def unrotate(v: np.ndarray) -> np.ndarray:
    """u = R^T v (H_64 is symmetric)."""
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    h = _hadamard64() / 8.0
    blocks = v.reshape(v.shape[:-1] + (d // 64, 64))
    return (np.einsum("ij,...bj->...bi", h, blocks) * rotation_signs()).reshape(v.shape)


# --------------------------------------------------------------------------
# O9: gain-shape scalar quantization                   [Method/4], [Findings/SQ]
# --------------------------------------------------------------------------
def gains_f32(var: np.ndarray) -> np.ndarray:
    """Per-bin gain stored in 32 bits: g = sqrt(variance), rounded to fp32.

    READING: [Method/4] factors out the l2 norm of each bin vector with 32
    side bits per bin; the stored value is the RMS norm |c| / sqrt(d), i.e.
    the l2 norm with the sqrt(d) folded into the unit-Gaussian table.
    """
    return np.sqrt(np.asarray(var, dtype=np.float64)).astype(np.float32)


def gains_absmax_f32(coef: np.ndarray, rotation: str = "none") -> np.ndarray:
    """Per-bin gain of the uniform and NormalFloat quantizers: the largest
    |value| of the bin vector (after the rotation when it is on), rounded to
    fp32, so the scaled values lie in [-1, 1].  READING: both quantizers
    scale by the absolute maximum, as those formats are defined."""
    c = np.asarray(coef, dtype=np.float64)
    if rotation == "hadamard":
        c = rotate(c)
    return np.max(np.abs(c), axis=-1).astype(np.float32)


def quantize(coef: np.ndarray, gains: np.ndarray, bits: np.ndarray,
             rotation: str = "none", kind: str = "lloyd_max") -> np.ndarray:
    """Cell index of every coefficient at its bin's bit width [Method/4].

    Decided in float32 (the kernel's precision): r = 1/g (0 when g == 0),
    u = fl32(c * r); with rotation="hadamard" the bin vector is rotated,
    v = fl32(R u) (R u in fp64 from the fp32 u); code = number of fp32
    thresholds <= the value (a value exactly on a threshold goes to the
    upper cell).  Bins with 0 bits get code 0 and are not stored.  Returns
    uint8 codes with the shape of ``coef``.
    """
    c32 = np.asarray(coef).astype(np.float32)
    g = np.asarray(gains, dtype=np.float32).reshape(c32.shape[:-1])
    b = np.asarray(bits).reshape(c32.shape[:-1]).astype(np.int64)
    with np.errstate(divide="ignore"):
        r = np.where(g > 0, np.float32(1.0) / np.where(g > 0, g, np.float32(1.0)),
                     np.float32(0.0)).astype(np.float32)
    u = (c32 * r[..., None]).astype(np.float32)
    if rotation == "hadamard":
        u = rotate(u.astype(np.float64)).astype(np.float32)
    codes = np.zeros(c32.shape, dtype=np.uint8)
    for nb in range(1, 9):
        sel = b == nb
        if not sel.any():
            continue
        _, thr = codebook_f32(nb, kind)
        codes[sel] = np.searchsorted(thr, u[sel], side="right").astype(np.uint8)
    return codes


def dequantize(codes: np.ndarray, gains: np.ndarray, bits: np.ndarray,
               rotation: str = "none", kind: str = "lloyd_max") -> np.ndarray:
    """c_hat = g * R^T level_b[code] (R = I without rotation); 0-bit bins
    reconstruct to exactly 0 [Method/dec]."""
    codes = np.asarray(codes)
    g = np.asarray(gains, dtype=np.float64).reshape(codes.shape[:-1])
    b = np.asarray(bits).reshape(codes.shape[:-1]).astype(np.int64)
    out = np.zeros(codes.shape, dtype=np.float64)
    for nb in range(1, 9):
        sel = b == nb
        if not sel.any():
            continue
        levels, _ = codebook(nb, kind)
        lv = levels[codes[sel].astype(np.int64)]
        if rotation == "hadamard":
            lv = unrotate(lv)
        out[sel] = g[sel][..., None] * lv
    return out


# --------------------------------------------------------------------------
# O10: the compressed record                          [Method/4] occupancy
# --------------------------------------------------------------------------
def _align256(n: int) -> int:
    return (n + 255) // 256 * 256


def record_layout(p: Params) -> dict:
    """Byte layout of one unit's record (all regions 256-byte aligned).

    gains  float32[n_bins]       the per-bin gain (the 32 side bits)
    bits   uint8[n_bins]         bits of each bin
    groups uint32[ceil(n/64)]    first bit-plane of bins 64g (the index)
    codes  uint64 words          bit-planes, T * head_dim bits in total
    READING: the page gives the occupancy (b_i * d + 32 bits per surviving
    bin plus a small index) but not the layout; this layout is ours.
    """
    nb = p.n_bins
    ng = (nb + 63) // 64
    code_bytes = total_bits(p) * p.head_dim // 8
    off_gains = 0
    off_bits = off_gains + _align256(4 * nb)
    off_groups = off_bits + _align256(nb)
    off_codes = off_groups + _align256(4 * ng)
    size = off_codes + _align256(code_bytes)
    return dict(gains=off_gains, bits=off_bits, groups=off_groups,
                codes=off_codes, code_bytes=code_bytes, n_groups=ng, size=size)


def pack_record(codes: np.ndarray, gains: np.ndarray, bits: np.ndarray,
                p: Params) -> np.ndarray:
    """Serialize one unit.  Bin i (flat order) starts at bit-plane
    P_i = sum_{k<i} b_k; its plane q (0 = least significant bit of the code)
    holds d bits at bit offset (P_i + q) * d of the codes region, bit j of
    the plane being bit q of code_j; 64-bit little-endian words.
    """
    lay = record_layout(p)
    d = p.head_dim
    rec = np.zeros(lay["size"], dtype=np.uint8)
    b = np.asarray(bits).ravel().astype(np.int64)
    if int(b.sum()) != total_bits(p):
        raise ValueError("bits do not sum to the budget")
    rec[lay["gains"]:lay["gains"] + 4 * p.n_bins] = \
        np.asarray(gains, dtype="<f4").ravel().view(np.uint8)
    rec[lay["bits"]:lay["bits"] + p.n_bins] = b.astype(np.uint8)
    start = np.concatenate([[0], np.cumsum(b)[:-1]]).astype(np.int64)
    grp = start[::64].astype("<u4")
    rec[lay["groups"]:lay["groups"] + 4 * lay["n_groups"]] = grp.view(np.uint8)
    c = np.asarray(codes).reshape(p.n_bins, d).astype(np.int64)
    bitstream = np.zeros(lay["code_bytes"] * 8, dtype=np.uint8)
    j = np.arange(d, dtype=np.int64)
    for q in range(int(b.max(initial=0))):
        sel = np.nonzero(b > q)[0]                     # bins that own plane q
        pos = ((start[sel] + q) * d)[:, None] + j[None, :]
        bitstream[pos] = ((c[sel] >> q) & 1).astype(np.uint8)
    # bit n of the stream is bit (n mod 8) of byte n // 8 (little-endian words)
    packed = np.packbits(bitstream, bitorder="little")
    rec[lay["codes"]:lay["codes"] + lay["code_bytes"]] = packed
    return rec


def unpack_record(rec: np.ndarray, p: Params):
    """Inverse of ``pack_record``: returns (codes uint8 (..., d), gains fp32, bits)."""
    lay = record_layout(p)
    d = p.head_dim
    rec = np.asarray(rec, dtype=np.uint8)
    gains = rec[lay["gains"]:lay["gains"] + 4 * p.n_bins].view("<f4").copy()
    b = rec[lay["bits"]:lay["bits"] + p.n_bins].astype(np.int64)
    start = np.concatenate([[0], np.cumsum(b)[:-1]]).astype(np.int64)
    stream = np.unpackbits(rec[lay["codes"]:lay["codes"] + lay["code_bytes"]],
                           bitorder="little").astype(np.int64)
    codes = np.zeros((p.n_bins, d), dtype=np.int64)
    j = np.arange(d, dtype=np.int64)
    for q in range(int(b.max(initial=0))):
        sel = np.nonzero(b > q)[0]
        pos = ((start[sel] + q) * d)[:, None] + j[None, :]
        codes[sel] |= stream[pos] << q
    shp = p.shape
    return (codes.astype(np.uint8).reshape(shp), gains.reshape(shp[:-1]),
            b.reshape(shp[:-1]))


# --------------------------------------------------------------------------
# O11: output rounding
# --------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits), to nearest even.

    Done directly from float64 (no intermediate float32, so no double
    rounding).  Returns float64 values that are exactly representable in
    bfloat16.  Values beyond the bfloat16 range are not expected here.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                        # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values that are exactly bfloat16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Whole codec                                          [Method/1-4], [Method/dec]
# --------------------------------------------------------------------------
def allocate_uniform(var: np.ndarray, budget_bits: int) -> np.ndarray:
    """Every bin gets the average budget: the page's "uniform allocation"
    comparison ("Main Findings", transform and allocation ablation)."""
    return np.full(np.asarray(var).size, int(budget_bits), dtype=np.int64)


def compress(x: np.ndarray, p: Params, axes=(0, 1, 2), alloc: str = "waterfill",
             rotation: str = "hadamard", quantizer: str = "lloyd_max") -> np.ndarray:
    """One unit: transform, variances, allocation, quantization, record.

    ``axes`` and ``alloc`` ("waterfill" or "uniform") select the page's
    ablations; the method is all three axes with water-filling.
    ``rotation`` is "hadamard" (the page's shared rotation, the method)
    or "none" (the identity, an ablation).  ``quantizer`` is "lloyd_max"
    (the method: RMS gain, Gaussian Lloyd-Max table) or one of the
    backends of [Findings/SQ], "uniform" or "nf" (absmax gain of every bin,
    the allocation unchanged).
    """
    x = np.asarray(x, dtype=np.float64).reshape(p.shape)
    coef = dct3_forward(x, axes)
    var = bin_variance(coef)
    if alloc == "uniform":
        bits = allocate_uniform(var, p.budget_bits).reshape(var.shape)
    else:
        bits = allocate_bits(var, total_bits(p), p.max_bits).reshape(var.shape)
    g = gains_f32(var) if quantizer == "lloyd_max" else gains_absmax_f32(coef, rotation)
    codes = quantize(coef, g, bits, rotation, quantizer)
    return pack_record(codes, g, bits, p)


def decompress(rec: np.ndarray, p: Params, out_dtype="bf16",
               axes=(0, 1, 2), rotation: str = "hadamard",
               quantizer: str = "lloyd_max") -> np.ndarray:
    """Unpack, dequantize, inverse transform, round [Method/dec].

    READING: the output is rounded to bfloat16 (nearest even) for a bf16
    cache, or to float32 for a float32 cache.
    """
    codes, g, b = unpack_record(rec, p)
    xr = dct3_inverse(dequantize(codes, g, b, rotation, quantizer), axes)
    if out_dtype == "bf16":
        return round_to_bf16(xr)
    if out_dtype == "f32":
        return xr.astype(np.float32).astype(np.float64)
    return xr


def roundtrip(x: np.ndarray, p: Params, out_dtype="bf16", axes=(0, 1, 2),
              alloc: str = "waterfill", rotation: str = "hadamard",
              quantizer: str = "lloyd_max"):
    rec = compress(x, p, axes, alloc, rotation, quantizer)
    return decompress(rec, p, out_dtype, axes, rotation, quantizer), rec


# --------------------------------------------------------------------------
# O12: metrics
# --------------------------------------------------------------------------
def mse(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.mean((a - b) ** 2))


def spectral_flatness(var: np.ndarray) -> float:
    """gamma = geometric mean / arithmetic mean of the bin variances
    (Theorem 1 of the page, [Contrib/2]); 1 for a flat spectrum."""
    v = np.asarray(var, dtype=np.float64).ravel()
    return float(np.exp(np.mean(np.log(v))) / np.mean(v))


def occupancy_bits(bits: np.ndarray, head_dim: int) -> int:
    """The page's occupancy count: sum over surviving bins of b_i * d + 32."""
    b = np.asarray(bits).ravel()
    return int(np.sum(b * head_dim) + 32 * np.count_nonzero(b))


def absmax_to_std(coef: np.ndarray) -> np.ndarray:
    """Per-bin max |c_j| over sqrt(mean c_j^2), the heavy-tail statistic of
    [Findings/SQ]; returns one value per bin (0-energy bins dropped)."""
    c = np.asarray(coef, dtype=np.float64)
    rms = np.sqrt(np.mean(c * c, axis=-1))
    am = np.max(np.abs(c), axis=-1)
    keep = rms > 0
    return am[keep] / rms[keep]


# --------------------------------------------------------------------------
# O13: serving capacity at equal HBM          [Findings/batch], [Method/1]
# --------------------------------------------------------------------------
def capacity_model(p: Params, layers: int, text_tokens: int, hbm_bytes: int,
                   weight_bytes: int, window_layers: int = 0,
                   reserve_bytes: int = 0) -> dict:
    """Per-request cache and maximum decoding batch, bf16 against coded.

    [Findings/batch] ("Main Findings", the bullet on batch and throughput at
    equal HBM): the per-request cache shrinks and the largest batch that fits
    beside the weights grows.  [Method/1]: text keys and values stay bf16.
    READING: a request is one sequence; each layer holds its text KV
    (text_tokens x K,V x kv_heads x head_dim bf16) and its visual K and V
    volumes, either bf16 or one record each; layers with sliding-window
    attention ("Future Directions") keep bf16 visual KV; the batch is the
    number of whole requests in the HBM left after the weights and a reserve.
    """
    text = text_tokens * layers * 2 * p.kv_heads * p.head_dim * 2
    unit_bf16 = p.n_entries * 2
    rec = record_layout(p)["size"]
    bf16 = text + layers * 2 * unit_bf16
    coded = text + (layers - window_layers) * 2 * rec + window_layers * 2 * unit_bf16
    free = max(hbm_bytes - weight_bytes - reserve_bytes, 0)
    return dict(request_bytes_bf16=bf16, request_bytes_coded=coded,
                batch_bf16=free // bf16, batch_coded=free // coded)


# --------------------------------------------------------------------------
# O14: attention over the decoded visual cache                 [Method/dec]
# --------------------------------------------------------------------------
def attend(k_rec: np.ndarray, v_rec: np.ndarray, p: Params, q: np.ndarray,
           scale: float, axes=(0, 1, 2), rotation: str = "hadamard",
           quantizer: str = "lloyd_max"):
    """One decoding step of attention over one unit pair's visual tokens.

    [Method/dec]: decoding reverses the codec, and the page allows it to run
    inside attention, reading only the records with no decoded cache written.
    This is the plain definition of what such a kernel returns, written on
    the decoded cache itself (fp64, no output rounding).
    READING: q holds one query per query head, shape (q_heads, head_dim),
    with grouped heads: query head r reads kv head r // (q_heads / kv_heads).
    The result is the softmax attention of each query over the S*H*W visual
    tokens of its kv head, out[r] = sum_t p_t v_t with
    p_t = exp(scale q_r . k_t - lse_r), and lse_r = log sum_t exp(scale q_r . k_t),
    which is what a caller needs to merge it with attention over the text
    tokens.
    """
    K = decompress(k_rec, p, None, axes, rotation, quantizer)
    V = decompress(v_rec, p, None, axes, rotation, quantizer)
    q = np.asarray(q, dtype=np.float64)
    qh = q.shape[0]
    rep = qh // p.kv_heads
    n = p.S * p.H * p.W
    out = np.zeros((qh, p.head_dim))
    lse = np.zeros(qh)
    for r in range(qh):
        h = r // rep
        k = K[:, :, :, h, :].reshape(n, p.head_dim)
        v = V[:, :, :, h, :].reshape(n, p.head_dim)
        s = scale * (k @ q[r])
        m = s.max()
        lse[r] = m + np.log(np.sum(np.exp(s - m)))
        out[r] = np.exp(s - lse[r]) @ v
    return out, lse
