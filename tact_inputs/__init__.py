"""Seeded synthetic KV-cache volumes for tests and the benchmark.

This module only draws inputs.  It holds none of the codec's arithmetic and
imports neither the oracle nor the HIP library, so both sides can be fed the
same tensors.

The caches the method was evaluated on (CT volumes and videos run through
medical and general VLMs) are not available here; these fields stand in for
them.  Each unit (one layer, one sequence, K or V) is a (S, H, W, kv_heads,
head_dim) volume drawn as a separable AR(1) Gaussian field: unit-variance
i.i.d. noise filtered along S, then H, then W with
    y_0 = e_0,   y_i = rho * y_{i-1} + sqrt(1 - rho^2) * e_i,
so the covariance is rho_S^|ds| rho_H^|dh| rho_W^|dw|; every (head, channel)
column is independent.  Heavy tails come from per-channel scales.  The field
is drawn in float32 with torch's generator on the requested device, then
rounded to the workload's dtype.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "unit_index", "unit_seed", "generate_unit",
           "generate_units"]


@dataclass(frozen=True)
class Workload:
    name: str
    S: int
    H: int
    W: int
    kv_heads: int
    head_dim: int
    layers: int
    batch: int                 # sequences per launch
    dtype: torch.dtype
    budgets: tuple             # average code bits per entry
    max_bits: int
    rho_s: float = 0.9
    rho_h: float = 0.9
    rho_w: float = 0.9
    rho_per_layer: tuple | None = None   # (lo, hi): one rho per layer, all axes
    scale: str = "student_t3"            # "spike" | "student_t3"
    spike_frac: float = 0.01
    spike_gain: float = 8.0
    scene_cuts: int = 0                  # restarts of the S recursion
    seed: int = 0
    workload_id: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def n_units(self) -> int:
        return self.layers * self.batch * 2

    @property
    def unit_shape(self):
        return (self.S, self.H, self.W, self.kv_heads, self.head_dim)

    @property
    def unit_entries(self) -> int:
        return self.S * self.H * self.W * self.kv_heads * self.head_dim


WORKLOADS = {
    # 1 layer, K and V, 256 tokens x 2 heads x 64, float32; rho 0.9 on all
    # three axes; 1% of the channels scaled x8; 1 bit/entry, cap 3 bits.
    "tiny": Workload("tiny", 4, 8, 8, 2, 64, layers=1, batch=1,
                     dtype=torch.float32, budgets=(1,), max_bits=3,
                     rho_s=0.9, rho_h=0.9, rho_w=0.9, scale="spike",
                     workload_id=0),
    # CT volume, 4B-class decoder: 34 layers, 32x16x16 tokens, 4 x 256.
    "ct4b": Workload("ct4b", 32, 16, 16, 4, 256, layers=34, batch=1,
                     dtype=torch.bfloat16, budgets=(1, 2, 4), max_bits=8,
                     rho_s=0.8, rho_h=0.92, rho_w=0.92, workload_id=1),
    # CT volume, 7B-class decoder: 28 layers, 64x16x16 tokens, 4 x 128,
    # 8 sequences per launch.
    "ct7b": Workload("ct7b", 64, 16, 16, 4, 128, layers=28, batch=8,
                     dtype=torch.bfloat16, budgets=(1,), max_bits=8,
                     rho_s=0.8, rho_h=0.92, rho_w=0.92, workload_id=2),
    # CT volume, 32B-class decoder: 64 layers, 64x24x24 tokens, 8 x 128;
    # one rho per layer drawn uniformly in [0.6, 0.95].
    "ct32b": Workload("ct32b", 64, 24, 24, 8, 128, layers=64, batch=1,
                      dtype=torch.bfloat16, budgets=(1,), max_bits=8,
                      rho_per_layer=(0.6, 0.95), workload_id=3),
    # Video: 28 layers, 64 frames of 14x14 tokens, 4 x 128, 16 sequences;
    # temporal rho 0.97, spatial 0.85, 3 scene cuts per sequence.
    "video": Workload("video", 64, 14, 14, 4, 128, layers=28, batch=16,
                      dtype=torch.bfloat16, budgets=(1, 2), max_bits=8,
                      rho_s=0.97, rho_h=0.85, rho_w=0.85, scene_cuts=3,
                      workload_id=4),
}


def unit_index(wl: Workload, layer: int, seq: int, kv: int) -> int:
    """Position of a unit in a launch: (layer, sequence, K=0/V=1), K/V fastest."""
    return (layer * wl.batch + seq) * 2 + kv


def unit_seed(wl: Workload, layer: int, seq: int, kv: int, salt: int = 0) -> int:
    """Substream seed keyed by (workload, sequence, layer, K/V)."""
    return (((wl.seed * 31 + wl.workload_id) * 4099 + layer) * 65537 + seq) * 4 + kv \
        + salt * 1_000_000_007


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _layer_rho(wl: Workload, layer: int) -> tuple:
    if wl.rho_per_layer is None:
        return wl.rho_s, wl.rho_h, wl.rho_w
    lo, hi = wl.rho_per_layer
    g = _gen("cpu", unit_seed(wl, layer, 0, 0, salt=1))
    r = lo + (hi - lo) * float(torch.rand((), generator=g, dtype=torch.float64))
    return r, r, r


def _scene_cuts(wl: Workload, seq: int) -> list:
    if wl.scene_cuts <= 0:
        return []
    g = _gen("cpu", unit_seed(wl, 0, seq, 0, salt=2))
    perm = torch.randperm(wl.S - 1, generator=g)[: wl.scene_cuts] + 1
    return sorted(int(v) for v in perm)


def _ar1_(y: torch.Tensor, dim: int, rho: float, restarts=()) -> None:
    """In place: AR(1) recursion along ``dim`` over i.i.d. unit noise ``y``."""
    a = float(rho)
    b = math.sqrt(max(0.0, 1.0 - a * a))
    n = y.shape[dim]
    rs = set(restarts)
    for i in range(1, n):
        if i in rs:
            continue                      # y_i = e_i: the recursion restarts
        cur = y.select(dim, i)
        cur.mul_(b).add_(y.select(dim, i - 1), alpha=a)


def generate_unit(wl: Workload, layer: int, seq: int, kv: int,
                  device="cpu", out: torch.Tensor | None = None) -> torch.Tensor:
    """One (S, H, W, kv_heads, head_dim) unit, deterministic in its key."""
    dev = torch.device(device)
    g = _gen(dev, unit_seed(wl, layer, seq, kv))
    y = torch.randn(wl.unit_shape, generator=g, device=dev, dtype=torch.float32)
    rs, rh, rw = _layer_rho(wl, layer)
    _ar1_(y, 0, rs, _scene_cuts(wl, seq))
    _ar1_(y, 1, rh)
    _ar1_(y, 2, rw)
    nch = wl.kv_heads * wl.head_dim
    gs = _gen("cpu", unit_seed(wl, layer, seq, kv, salt=3))
    if wl.scale == "spike":
        k = max(1, round(wl.spike_frac * nch))
        idx = torch.randperm(nch, generator=gs)[:k]
        sc = torch.ones(nch, dtype=torch.float32)
        sc[idx] = wl.spike_gain
    else:                                 # |t| with t ~ Student-t(3)
        z = torch.randn(nch, generator=gs, dtype=torch.float64)
        chi2 = (torch.randn(nch, 3, generator=gs, dtype=torch.float64) ** 2).sum(1)
        sc = (z / torch.sqrt(chi2 / 3.0)).abs().to(torch.float32)
    y.mul_(sc.to(dev).view(1, 1, 1, wl.kv_heads, wl.head_dim))
    if out is None:
        return y.to(wl.dtype)
    out.copy_(y)
    return out


def generate_units(wl: Workload, units=None, device="cpu") -> torch.Tensor:
    """A launch's worth of units, shape (n_units, S, H, W, kv_heads, head_dim).

    ``units`` is a list of (layer, seq, kv) keys; by default every unit of
    the workload in launch order.
    """
    if units is None:
        units = [(l, s, k) for l in range(wl.layers) for s in range(wl.batch)
                 for k in range(2)]
    out = torch.empty((len(units),) + wl.unit_shape, dtype=wl.dtype,
                      device=torch.device(device))
    for i, (l, s, k) in enumerate(units):
        generate_unit(wl, l, s, k, device=device, out=out[i])
    return out
