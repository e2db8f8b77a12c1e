"""tact_roundtrip_noalloc: the round trip on the library's static per-GPU
workspace, for callers that cannot allocate device memory.  It must give
tact_roundtrip's results bit for bit, on consecutive calls of different sizes
(the array keeps the previous call's contents), and refuse geometries whose
single unit does not fit the array before touching the GPU."""
import ctypes

import pytest
import torch

from kv_cache_compression_tact_amd import TactParams, lib
from tact_inputs import WORKLOADS, generate_units


def say(*a):
    print(*a, flush=True)


def test_noalloc_refuses_units_larger_than_the_static_workspace():
    L = lib()
    p = TactParams()
    # 64 x 32 x 32 x 8 x 128: 2^26 entries, 256 MiB of fp32 volume per unit
    L.tact_params_init(ctypes.byref(p), 64, 32, 32, 8, 128, 1)
    fake = ctypes.c_void_p(1 << 30)
    assert L.tact_workspace_bytes(ctypes.byref(p), 1) > (192 << 20)
    assert L.tact_roundtrip_noalloc(ctypes.byref(p), 1, fake, 1 << 26, ctypes.c_void_p(1 << 40),
                                    1 << 26, None, None) == 2
    assert b"static workspace" in L.tact_last_error()
    # the largest workload unit fits
    q = TactParams()
    L.tact_params_init(ctypes.byref(q), 64, 24, 24, 8, 128, 1)
    assert L.tact_workspace_bytes(ctypes.byref(q), 1) <= (192 << 20)
    assert L.tact_roundtrip_noalloc(ctypes.byref(q), 0, None, 0, None, 0, None, None) == 0


@pytest.mark.gpu
def test_noalloc_matches_roundtrip_on_consecutive_calls():
    import kv_cache_compression_tact_amd as tact
    # first call: two full-size ct32b units (one unit per chunk of the array)
    wl = WORKLOADS["ct32b"]
    say("noalloc call 1: ct32b, 2 units")
    x = generate_units(wl, units=[(0, 0, 0), (0, 0, 1)], device="cuda")
    ref_out, ref_rec = tact.roundtrip(x, 1, wl.max_bits)
    out = torch.empty_like(x)
    rec = torch.empty_like(ref_rec)
    tact.roundtrip_noalloc(x, 1, wl.max_bits, out=out, records=rec)
    torch.cuda.synchronize()
    assert torch.equal(rec, ref_rec)
    assert torch.equal(out, ref_out)
    del x, out, rec, ref_out, ref_rec
    torch.cuda.empty_cache()
    # second call, smaller: a ragged geometry, records kept in the array
    say("noalloc call 2: 5 x 7 x 9 x 3 x 64, 3 units, records in the static workspace")
    gen = torch.Generator(device="cpu").manual_seed(31)
    y = torch.randn((3, 5, 7, 9, 3, 64), generator=gen).to(torch.bfloat16).cuda()
    ref_out, _ = tact.roundtrip(y, 2)
    out = torch.empty_like(y)
    tact.roundtrip_noalloc(y, 2, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    # in place, with the records kept by the caller
    z = y.clone()
    rec = torch.empty((3, tact.Geometry.of(y, 2).record_bytes()), dtype=torch.uint8, device="cuda")
    tact.roundtrip_noalloc(z, 2, out=z, records=rec)
    torch.cuda.synchronize()
    assert torch.equal(z, ref_out)
    # the per-axis path (W beyond 32) and fp32 caches share the array too
    for shape, dt in (((3, 5, 40, 1, 128), torch.bfloat16), ((2, 6, 7, 2, 64), torch.float32)):
        say("noalloc:", shape, dt)
        z = torch.randn((2,) + shape, generator=gen).to(dt).cuda()
        ref_out, ref_rec = tact.roundtrip(z, 1)
        out = torch.empty_like(z)
        rec = torch.empty_like(ref_rec)
        tact.roundtrip_noalloc(z, 1, out=out, records=rec)
        torch.cuda.synchronize()
        assert torch.equal(rec, ref_rec) and torch.equal(out, ref_out)
    say("noalloc: equal to tact_roundtrip on every call")


@pytest.mark.gpu
def test_noalloc_roundtrip_captured_in_a_graph():
    # The callers this entry point serves include code under HIP graph
    # capture: the captured call allocates nothing and records only kernel
    # launches, so every replay (with the program's own work between them)
    # gives the eager results.
    import kv_cache_compression_tact_amd as tact
    gen = torch.Generator(device="cpu").manual_seed(37)
    x = torch.randn((3, 5, 7, 9, 3, 64), generator=gen).to(torch.bfloat16).cuda()
    ref_out, ref_rec = tact.roundtrip(x, 2)
    out = torch.empty_like(x)
    rec = torch.empty_like(ref_rec)
    tact.roundtrip_noalloc(x, 2, out=out, records=rec)      # eager: the array's address is known
    torch.cuda.synchronize()
    assert torch.equal(rec, ref_rec) and torch.equal(out, ref_out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tact.roundtrip_noalloc(x, 2, out=out, records=rec)
    for replay in range(3):
        out.zero_()
        rec.zero_()
        graph.replay()
        torch.cuda.synchronize()
        say("noalloc graph replay", replay)
        assert torch.equal(rec, ref_rec) and torch.equal(out, ref_out)
    # eager calls between replays leave the captured call's results unchanged
    y = torch.randn(tuple(x.shape), generator=gen).to(torch.bfloat16).cuda()
    tact.roundtrip_noalloc(y, 1, out=torch.empty_like(y))
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(rec, ref_rec) and torch.equal(out, ref_out)
