#!/usr/bin/env python3
"""Throughput of the TACT-KV codec on one MI355X.

A step is one pass of the whole codec over one launch's worth of synthetic
KV cache resident in HBM: tact_compress over every unit of the workload,
then tact_decompress of every record.  Printed as ONE JSON line:

  value     GB/s of bf16 KV compressed and decompressed: input bytes of all
            units divided by (compress + decompress) time
  roofline  HBM roofline of the codec call that dominates the step:
            algorithmic bytes per call (what the call must read and write:
            2 B in / B/8 + 5/d out for compress, the reverse for
            decompress, per entry) over its average duration, timed with
            HIP events on the stream the library launches on
  cpu_baseline  the plain CPU oracle timed on a bounded sample (layer 0,
            sequence 0, K and V) of the same workload on the host cores

    python bench.py [--steps K] [--warmup W] [--workload ct32b] [--budget 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ct32b",
                    choices=["tiny", "ct4b", "ct7b", "ct32b", "video"])
    ap.add_argument("--budget", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=2,
                    help="units in the oracle's timed sample")
    ap.add_argument("--attend", action="store_true",
                    help="time decoding fused into attention (tact_attend) over every "
                         "layer and sequence of the workload instead of the codec")
    ap.add_argument("--ablations", action="store_true",
                    help="reconstruction error of the page's ablations (axes, allocation, "
                         "rotation, quantizer backends) on the GPU, and Theorem 1's closure")
    ap.add_argument("--ablation-units", type=int, default=8,
                    help="units of the workload used by --ablations")
    ap.add_argument("--q-per-kv", type=int, default=4,
                    help="query heads per kv head for --attend")
    ap.add_argument("--ws-units", type=int, default=None,
                    help="give the codec a workspace for this many units, so the batch "
                         "runs in chunks of that size (default: the whole batch at once)")
    ap.add_argument("--calibrate-bandwidth", action="store_true",
                    help="only measure this device's plain read-only, write-only and copy "
                         "rates on 8 GiB buffers (torch's kernels)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times): the "
                         "reference for scaling the HBM byte counters of a profile")
    return ap.parse_args()


def calibrate_copy():
    """Three copies of exactly 1 GiB between device buffers, nothing else,
    each timed with HIP events: the reference for scaling the byte counters
    of a profile, and the plain copy rate of this device."""
    dev = torch.device("cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        b.synchronize()
        ms.append(a.elapsed_time(b))
    best = min(ms)
    print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                      "repeats": 3, "ms": [round(m, 4) for m in ms],
                      "copy_GBs_read_plus_write": round(2 * (1 << 30) / (best * 1e-3) / 1e9, 1)}),
          flush=True)


def calibrate_bandwidth():
    """The plain HBM rates of this device with torch's own kernels on 8 GiB
    buffers (far beyond the 256 MB Infinity Cache): read-only (a sum),
    write-only (a fill) and a copy (read + write), three repeats each, the
    best taken.  The reference rates the codec's kernels are compared with."""
    dev = torch.device("cuda:0")
    n = 1 << 31                                   # 8 GiB of fp32
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def best_ms(fn):
        ms = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        return min(ms)

    nbytes = 4 * n
    torch.cuda.synchronize()
    r = best_ms(lambda: x.sum())
    w = best_ms(lambda: y.fill_(2.0))
    c = best_ms(lambda: y.copy_(x))
    print(json.dumps({"calibration": "bandwidth", "bytes": nbytes,
                      "read_only_GBs": round(nbytes / (r * 1e-3) / 1e9, 1),
                      "write_only_GBs": round(nbytes / (w * 1e-3) / 1e9, 1),
                      "copy_GBs_read_plus_write": round(2 * nbytes / (c * 1e-3) / 1e9, 1),
                      "ms": {"read": round(r, 3), "write": round(w, 3), "copy": round(c, 3)}}),
          flush=True)


def cpu_baseline(wl, budget, n_units):
    """Time the oracle (as it stands) on a bounded sample of the workload."""
    import numpy as np

    import oracle as O
    from tact_inputs import generate_unit
    keys = [(0, 0, 0), (0, 0, 1), (1, 0, 0), (1, 0, 1)][:n_units]
    keys = [k for k in keys if k[0] < wl.layers]
    xs = [generate_unit(wl, *k).float().numpy().astype(np.float64) for k in keys]
    p = O.Params(*wl.unit_shape, budget_bits=budget, max_bits=wl.max_bits)
    od = "bf16" if wl.dtype == torch.bfloat16 else "f32"
    t0 = time.perf_counter()
    for x in xs:
        O.decompress(O.compress(x, p), p, od)
    dt = time.perf_counter() - t0
    nbytes = len(xs) * wl.unit_entries * (2 if wl.dtype == torch.bfloat16 else 4)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = 1
    cores = len(os.sched_getaffinity(0))
    names = {(0, 0, 0): "layer 0 K", (0, 0, 1): "layer 0 V", (1, 0, 0): "layer 1 K",
             (1, 0, 1): "layer 1 V"}
    per_unit = dt / len(xs)
    return {
        "value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores,
        "kind": "oracle",
        "sample": f"{len(xs)} units ({', '.join(names[k] for k in keys)}; sequence 0) of "
                  f"{wl.name}, compress+decompress in {dt:.2f} s; BLAS threads {threads}",
        "blas_threads": int(threads),
        "extrapolated_full_config_s": round(per_unit * wl.n_units, 1),
        "extrapolated_note": f"linear in units: {per_unit:.2f} s per unit x {wl.n_units} units "
                             "(extrapolated, not measured)",
    }


def measured_traffic(workload: str):
    """HBM bytes per codec call from the committed counter summary, or None.

    profiles/codec_<workload>_hbm_traffic.md ends with a traffic-record line
    written from two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE)
    scaled by a copy-kernel calibration.  It is used only while the kernel
    sources still hash to the value recorded with the counters.
    """
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"codec_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("traffic-record:"):
            rec = json.loads(line.split(":", 1)[1])
    if rec is None:
        return None
    csrc = os.path.join(root, "kv_cache_compression_tact_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".cpp", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    if h.hexdigest() != rec.get("source_sha256"):
        return None
    return rec


def bench_ablations(args, tact, wl, budget, g, x):
    """Relative reconstruction error ||x_hat - x||^2 / ||x||^2 of the codec
    and of the page's ablations ("Main Findings": fewer transform axes,
    uniform allocation, the quantizer backends; and the rotation), all run on
    the GPU over the first units of the workload; and Theorem 1's closure:
    the measured distortion ratio of uniform to water-filling allocation
    beside 1/gamma, gamma the spectral flatness (geometric over arithmetic
    mean) of each unit's bin variances."""
    n = min(args.ablation_units, x.shape[0])
    xs = x[:n].contiguous()
    ref = xs.float()
    energy = float((ref * ref).sum())

    def err(**kw):
        out, _ = tact.roundtrip(xs, budget, wl.max_bits, keep_records=False, **kw)
        return float(((out.float() - ref) ** 2).sum()) / energy

    variants = {
        "method (3-axis DCT, water-filling, rotation, Lloyd-Max)": {},
        "2-axis DCT (H, W)": {"axes": tact.AXIS_H | tact.AXIS_W},
        "2-axis DCT (S, W)": {"axes": tact.AXIS_S | tact.AXIS_W},
        "1-axis DCT (S)": {"axes": tact.AXIS_S},
        "no transform": {"axes": tact.AXES_NONE},
        "uniform allocation": {"alloc_mode": tact.ALLOC_UNIFORM},
        "no rotation": {"rotation": tact.ROTATION_NONE},
        "symmetric uniform quantizer": {"quantizer": tact.QUANT_UNIFORM},
        "NormalFloat quantizer": {"quantizer": tact.QUANT_NF},
        "symmetric uniform quantizer, no rotation": {"quantizer": tact.QUANT_UNIFORM,
                                                     "rotation": tact.ROTATION_NONE},
        "NormalFloat quantizer, no rotation": {"quantizer": tact.QUANT_NF,
                                               "rotation": tact.ROTATION_NONE},
    }
    res = {name: round(err(**kw), 6) for name, kw in variants.items()}
    # Theorem 1: D_uniform / D_waterfill against 1 / gamma, per unit
    var = tact.dbg_bin_variance(xs.contiguous(), g).double().reshape(n, -1).clamp_min(1e-300)
    gamma = torch.exp(torch.log(var).mean(1)) / var.mean(1)
    out_w, _ = tact.roundtrip(xs, budget, wl.max_bits, keep_records=False)
    out_u, _ = tact.roundtrip(xs, budget, wl.max_bits, keep_records=False,
                              alloc_mode=tact.ALLOC_UNIFORM)
    dims = tuple(range(1, xs.dim()))
    d_w = ((out_w.float() - ref) ** 2).sum(dims).double()
    d_u = ((out_u.float() - ref) ** 2).sum(dims).double()
    closure = [{"unit": u, "inv_gamma": round(float(1 / gamma[u]), 3),
                "measured_ratio": round(float(d_u[u] / d_w[u]), 3)} for u in range(n)]
    line = {
        "metric": "relative reconstruction error of the codec and its ablations (GPU)",
        "value": res["method (3-axis DCT, water-filling, rotation, Lloyd-Max)"],
        "unit": "||x_hat - x||^2 / ||x||^2", "higher_is_better": False, "n_gpus": 1,
        "data": "synthetic",
        "config": {"workload": wl.name, "units": n, "unit_shape": list(wl.unit_shape),
                   "budget_bits": budget},
        "ablations": res, "theorem1_closure": closure,
    }
    print(json.dumps(line), flush=True)


def bench_attend(args, tact, wl, budget, g, x):
    """One decoding step of attention over the visual KV of every layer and
    sequence of the workload (one query per query head), read straight from
    the K and V records by tact_attend.  For reference the same records are
    decompressed to the bf16 cache with tact_decompress, which a path that
    materializes the cache must do before its attention reads it."""
    dev = x.device
    U = wl.n_units
    pairs = U // 2
    rec = tact.compress(x, budget, wl.max_bits)
    krec, vrec = rec[0::2].contiguous(), rec[1::2].contiguous()
    del x
    qh = args.q_per_kv * wl.kv_heads
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    q = torch.randn((pairs, qh, wl.head_dim), generator=gen, device=dev, dtype=torch.float32)
    ws = tact.attend_workspace(g, pairs, qh, dev)
    out_cache = torch.empty((U,) + g.unit_shape, dtype=g.dtype, device=dev)
    dws = tact.workspace(g, U, dev)
    stream = torch.cuda.current_stream()
    scale = 1.0 / wl.head_dim ** 0.5

    def timed(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    att = lambda: tact.attend(krec, vrec, g, q, scale, ws=ws)
    dec = lambda: tact.decompress(rec, g, out=out_cache, ws=dws)
    for _ in range(args.warmup):
        att()
        dec()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_att = timed(att, args.steps)
    elapsed = time.perf_counter() - t0
    t_dec = timed(dec, args.steps)
    ms_att = sum(t_att) / len(t_att)
    ms_dec = sum(t_dec) / len(t_dec)
    read = 2 * pairs * g.record_bytes()
    line = {
        "metric": "decode-attention step over the coded visual KV (tact_attend), ms",
        "value": round(ms_att, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "pairs": pairs, "q_heads": qh,
                   "unit_shape": list(wl.unit_shape), "budget_bits": budget},
        "record_bytes_read": read,
        "record_read_GBs": round(read / (ms_att * 1e-3) / 1e9, 2),
        "ms_decompress_same_records": round(ms_dec, 4),
        "speedup_vs_decompress": round(ms_dec / ms_att, 2),
    }
    print(json.dumps(line), flush=True)


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the codec is "
              "per layer, per sequence and needs no exchange between GPUs; run one process "
              "per GPU on its own share of the units.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate_bandwidth:
        calibrate_bandwidth()
        return
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import kv_cache_compression_tact_amd as tact
    from tact_inputs import WORKLOADS, generate_units

    wl = WORKLOADS[args.workload]
    budget = args.budget if args.budget is not None else wl.budgets[0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {wl.name}: {wl.n_units} units of {wl.unit_shape} "
          f"{wl.dtype}", file=sys.stderr, flush=True)
    x = generate_units(wl, device=dev)
    g = tact.Geometry(*wl.unit_shape, budget_bits=budget, max_bits=wl.max_bits,
                      dtype=wl.dtype)
    U = wl.n_units
    if args.attend:
        bench_attend(args, tact, wl, budget, g, x)
        return
    if args.ablations:
        bench_ablations(args, tact, wl, budget, g, x)
        return
    rec = torch.empty((U, g.record_bytes()), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    chunk = U if args.ws_units is None else max(1, min(args.ws_units, U))
    ws = tact.workspace(g, chunk, dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
          for _ in range(args.steps)]

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        tact.compress(x, budget, wl.max_bits, records=rec, ws=ws)
        if e is not None:
            e[1].record(stream)
        tact.decompress(rec, g, out=out, ws=ws)
        if e is not None:
            e[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    t_c = sorted(e[0].elapsed_time(e[1]) for e in ev)
    t_d = sorted(e[1].elapsed_time(e[2]) for e in ev)
    med = lambda v: v[len(v) // 2]
    ms_c, ms_d = sum(t_c) / len(t_c), sum(t_d) / len(t_d)
    es = 2 if wl.dtype == torch.bfloat16 else 4
    in_bytes = U * wl.unit_entries * es
    d = wl.head_dim
    # algorithmic bytes per entry: compress reads the cache and writes the
    # codes and side info; decompress reads those and writes the cache
    side = (budget / 8.0 + 5.0 / d)
    alg_c = U * wl.unit_entries * (es + side)
    alg_d = U * wl.unit_entries * (side + es)
    ms_step = elapsed * 1e3 / args.steps
    value = in_bytes / (elapsed / args.steps) / 1e9
    dom, alg, ms = ("tact_compress", alg_c, ms_c) if ms_c >= ms_d else \
        ("tact_decompress", alg_d, ms_d)
    achieved = alg / (ms * 1e-3) / 1e9
    roofline_step = (alg_c + alg_d) / ((ms_c + ms_d) * 1e-3) / 1e9
    # the counter record was taken on the whole batch in one chunk
    tr = measured_traffic(wl.name) if budget == wl.budgets[0] and chunk == U else None
    traffic = None
    if tr is not None:
        traffic = tr["compress_bytes"] if dom == "tact_compress" else tr["decompress_bytes"]
    line = {
        "metric": "KV codec GB/s (compress+decompress, bf16 in) and % of HBM roofline at 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "units": U, "unit_shape": list(wl.unit_shape),
                   "arithmetic": "fp32 accumulation, split-fp16 matrix-core products",
                   "cache_dtype": str(wl.dtype).replace("torch.", ""),
                   "budget_bits": budget, "max_bits": wl.max_bits,
                   "rotation": "hadamard" if g.rotation else "none",
                   "input_bytes": in_bytes, "units_per_chunk": chunk},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": int(alg),
                     "step_frac": round(roofline_step / HBM_PEAK_GBS, 4)},
        "ms_compress": round(ms_c, 4), "ms_decompress": round(ms_d, 4),
        "ms_compress_median": round(med(t_c), 4), "ms_decompress_median": round(med(t_d), 4),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, budget, args.cpu_units)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
