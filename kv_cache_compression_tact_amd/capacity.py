"""Serving capacity with TACT-KV-coded visual caches at equal HBM.

The page "TACT-KV: Tri-Axis Cosine Transform for Compressing Volumetric KV
Caches in Medical VLMs" reports, in "Main Findings", how much the per-request
cache shrinks and how far the maximum decoding batch grows when the visual
KV is coded; "Methodology in Plain English", stage 1, keeps the text keys and
values in bf16, and "Future Directions" notes that sliding-window attention
layers were left in bf16.  This module turns the library's record sizes into
that capacity figure for a given model and GPU.

Per request (one sequence):
  text KV    text_tokens x layers x 2 (K, V) x kv_heads x head_dim x 2 bytes;
  visual KV  for each of the `layers - window_layers` coded layers, two codec
             records (K and V, `tact_record_bytes` each); for each window
             layer the bf16 volumes, 2 x S*H*W*kv_heads*head_dim x 2 bytes.
The maximum decoding batch is the number of whole requests that fit in the
HBM left after the weights and a reserve.  Activations and allocator slack
belong in the reserve.
"""
from __future__ import annotations

import argparse
from dataclasses import dataclass

from . import Geometry

BF16_BYTES = 2


@dataclass(frozen=True)
class ServingModel:
    """A decoder and its visual grid.  Sizes in bytes."""
    layers: int
    kv_heads: int
    head_dim: int
    S: int
    H: int
    W: int
    text_tokens: int
    weight_bytes: int
    hbm_bytes: int = 288 * 10**9         # one MI355X
    window_layers: int = 0               # layers whose visual KV stays bf16
    reserve_bytes: int = 0
    budget_bits: int = 1
    max_bits: int = 8

    def __post_init__(self):
        if not 0 <= self.window_layers <= self.layers:
            raise ValueError("window_layers must be in 0..layers")
        if min(self.layers, self.kv_heads, self.head_dim, self.S, self.H, self.W) < 1:
            raise ValueError("layers, kv_heads, head_dim and the grid must be positive")
        if min(self.text_tokens, self.weight_bytes, self.reserve_bytes) < 0:
            raise ValueError("text_tokens, weight_bytes and reserve_bytes must be >= 0")


def text_kv_bytes(m: ServingModel) -> int:
    return m.text_tokens * m.layers * 2 * m.kv_heads * m.head_dim * BF16_BYTES


def visual_unit_bf16_bytes(m: ServingModel) -> int:
    return m.S * m.H * m.W * m.kv_heads * m.head_dim * BF16_BYTES


def record_bytes(m: ServingModel) -> int:
    """Bytes of one coded unit (the library's record size)."""
    return Geometry(m.S, m.H, m.W, m.kv_heads, m.head_dim, m.budget_bits,
                    m.max_bits).record_bytes()


def request_bytes(m: ServingModel, coded: bool) -> int:
    visual_bf16 = 2 * visual_unit_bf16_bytes(m)
    if not coded:
        return text_kv_bytes(m) + m.layers * visual_bf16
    coded_layers = m.layers - m.window_layers
    return (text_kv_bytes(m) + coded_layers * 2 * record_bytes(m)
            + m.window_layers * visual_bf16)


def max_batch(m: ServingModel, per_request: int) -> int:
    free = m.hbm_bytes - m.weight_bytes - m.reserve_bytes
    return max(free, 0) // per_request


def capacity(m: ServingModel) -> dict:
    """Per-request cache bytes and maximum batch, bf16 against coded."""
    bf16 = request_bytes(m, coded=False)
    coded = request_bytes(m, coded=True)
    b0, b1 = max_batch(m, bf16), max_batch(m, coded)
    return {
        "request_bytes_bf16": bf16,
        "request_bytes_coded": coded,
        "cache_ratio": bf16 / coded,
        "batch_bf16": b0,
        "batch_coded": b1,
        "batch_gain": (b1 / b0) if b0 else float("inf"),
    }


def _main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--layers", type=int, required=True)
    ap.add_argument("--kv-heads", type=int, required=True)
    ap.add_argument("--head-dim", type=int, required=True)
    ap.add_argument("--grid", type=int, nargs=3, metavar=("S", "H", "W"), required=True)
    ap.add_argument("--text-tokens", type=int, default=512)
    ap.add_argument("--weights-gb", type=float, required=True)
    ap.add_argument("--hbm-gb", type=float, default=288.0)
    ap.add_argument("--window-layers", type=int, default=0)
    ap.add_argument("--reserve-gb", type=float, default=0.0)
    ap.add_argument("--budget", type=int, default=1)
    a = ap.parse_args()
    m = ServingModel(a.layers, a.kv_heads, a.head_dim, *a.grid, a.text_tokens,
                     int(a.weights_gb * 1e9), int(a.hbm_gb * 1e9), a.window_layers,
                     int(a.reserve_gb * 1e9), a.budget)
    for k, v in capacity(m).items():
        print(f"{k:20s} {v}")


if __name__ == "__main__":
    _main()
