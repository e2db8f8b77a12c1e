"""The C ABI without a GPU: the library loads, exports every function that
include/*.h declares, and rejects invalid calls before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

import kv_cache_compression_tact_amd as tact
from kv_cache_compression_tact_amd import TactParams, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("tact.h", "tact_debug.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(tact_[a-z0-9_]+)\s*\(", src))
    return names


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"tact_compress", "tact_decompress", "tact_roundtrip"} <= names
    for n in sorted(names):
        assert hasattr(lib(), n), n
    assert names == set(tact.EXPORTED)


def _params(**kw):
    p = TactParams()
    lib().tact_params_init(ctypes.byref(p), 4, 8, 8, 2, 64, 1)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_params_init_defaults():
    p = _params()
    assert (p.max_bits, p.dtype, p.axes, p.alloc_mode, p.rotation) == (8, 0, 7, 0, 1)


def test_record_bytes_matches_layout():
    p = _params(max_bits=3, dtype=1)
    # 512 bins: gains 2048, bits 512, groups 8*4 -> 256, codes 512*64/8 = 4096
    assert lib().tact_record_bytes(ctypes.byref(p)) == 2048 + 512 + 256 + 4096
    from oracle import Params, record_layout
    for geo in [(64, 24, 24, 8, 128, 1), (32, 16, 16, 4, 256, 4), (3, 5, 7, 1, 64, 2)]:
        q = _params(S=geo[0], H=geo[1], W=geo[2], kv_heads=geo[3], head_dim=geo[4],
                    budget_bits=geo[5])
        assert lib().tact_record_bytes(ctypes.byref(q)) == \
            record_layout(Params(*geo, max_bits=8))["size"]


@pytest.mark.parametrize("field,value,status", [
    ("S", 0, 2), ("H", 65, 2), ("W", -1, 2), ("kv_heads", 0, 2), ("head_dim", 96, 2),
    ("max_bits", 0, 1), ("max_bits", 9, 1), ("budget_bits", 9, 1), ("budget_bits", -1, 1),
    ("dtype", 5, 1), ("axes", -1, 1), ("axes", 8, 1), ("alloc_mode", 2, 1),
    ("rotation", 2, 1), ("rotation", -1, 1),
])
def test_invalid_params_rejected(field, value, status):
    p = _params(**{field: value})
    assert lib().tact_record_bytes(ctypes.byref(p)) == 0
    assert lib().tact_workspace_bytes(ctypes.byref(p), 4) == 0
    fake = ctypes.c_void_p(1 << 20)
    st = lib().tact_compress(ctypes.byref(p), 1, fake, 32768, fake, fake, 1 << 30, None)
    assert st == status
    assert len(lib().tact_last_error()) > 0


def test_no_transform_axes_accepted():
    # axes = 0: the no-transform ablation (tokens coded as they are)
    p = _params(axes=0)
    assert lib().tact_record_bytes(ctypes.byref(p)) == lib().tact_record_bytes(ctypes.byref(_params()))
    assert lib().tact_workspace_bytes(ctypes.byref(p), 4) > 0


def _padded_unit_bytes(S, H, W, kv_heads, head_dim):
    pad = lambda n: 16 if n <= 16 else 32 if n <= 32 else 64
    return 4 * pad(S) * pad(H) * pad(W) * kv_heads * head_dim


@pytest.mark.parametrize("shape,ok", [
    ((64, 64, 64, 16, 64), True),     # 2^28 entries, padded 2^30 bytes: the largest unit
    ((64, 64, 64, 32, 64), False),    # 2^29 entries: fp32 volume 2^31 bytes
    ((64, 64, 64, 64, 64), False),
    ((40, 20, 18, 32, 128), True),    # ragged on every axis, padded exactly 2^30
    ((33, 32, 32, 32, 128), True),    # S pads to 64: 2^30
    ((33, 33, 32, 32, 128), False),   # H pads to 64 too: 2^31, though only 2^27.1 entries
    ((2, 64, 64, 64, 64), True),      # S pads 2 -> 16: 2^30
    ((2, 64, 64, 64, 128), False),    # 2^27 entries, but padded 2^31 (rows past S would wrap)
    ((1, 1, 1, 64, 256), True),       # degenerate grid
])
def test_unit_size_cap(shape, ok):
    # the padded fp32 unit (each grid axis rounded up to 16, 32 or 64) is at
    # most 2^30 bytes; the worked sizes above are computed by hand
    assert (_padded_unit_bytes(*shape) <= 1 << 30) == ok
    S, H, W, kv, d = shape
    p = _params(S=S, H=H, W=W, kv_heads=kv, head_dim=d)
    assert (lib().tact_record_bytes(ctypes.byref(p)) > 0) == ok
    if not ok:
        fake = ctypes.c_void_p(1 << 20)
        assert lib().tact_compress(ctypes.byref(p), 1, fake, 1 << 31, fake, fake, 1 << 40,
                                   None) == 2
        assert "padded" in lib().tact_last_error().decode()


def test_null_and_misaligned_pointers_rejected():
    p = _params()
    ws = lib().tact_workspace_bytes(ctypes.byref(p), 2)
    assert ws > 0
    fake = ctypes.c_void_p(1 << 20)
    L = lib()
    assert L.tact_compress(ctypes.byref(p), 2, None, 32768, fake, fake, ws, None) == 1
    assert L.tact_compress(ctypes.byref(p), 2, ctypes.c_void_p((1 << 20) + 2), 32768, fake,
                           fake, ws, None) == 1
    assert L.tact_compress(ctypes.byref(p), 2, fake, 32768, None, fake, ws, None) == 1
    assert L.tact_compress(ctypes.byref(p), 2, fake, 32768, ctypes.c_void_p((1 << 20) + 16),
                           fake, ws, None) == 1
    # unit stride below the unit size or not a multiple of 8
    assert L.tact_compress(ctypes.byref(p), 2, fake, 32767, fake, fake, ws, None) == 1
    assert L.tact_compress(ctypes.byref(p), 2, fake, 32772, fake, fake, ws, None) == 1
    # workspace missing / too small: it must hold at least one unit (a
    # smaller workspace than tact_workspace_bytes(p, n) splits the batch)
    ws1 = L.tact_workspace_bytes(ctypes.byref(p), 1)
    assert 0 < ws1 < ws
    kv, rec, wsp = (ctypes.c_void_p(a << 30) for a in (1, 2, 3))   # disjoint fake buffers
    assert L.tact_compress(ctypes.byref(p), 2, kv, 32768, rec, None, ws, None) == 3
    assert L.tact_compress(ctypes.byref(p), 2, kv, 32768, rec, wsp, ws1 - 1, None) == 3
    assert L.tact_decompress(ctypes.byref(p), 2, rec, kv, 32768, wsp, ws1 - 1, None) == 3
    assert L.tact_compress(ctypes.byref(p), -1, kv, 32768, rec, wsp, ws, None) == 1
    # overlapping but distinct in/out for the round trip
    assert L.tact_roundtrip(ctypes.byref(p), 2, kv, 32768,
                            ctypes.c_void_p((1 << 30) + 4096), 32768, None, wsp, ws,
                            None) == 1
    # in place with unequal strides: a later chunk's input would be overwritten
    assert L.tact_roundtrip(ctypes.byref(p), 2, kv, 32768, kv, 65536, None, wsp, ws, None) == 1
    assert b"equal unit strides" in L.tact_last_error()
    # records over the cache, the workspace over the records
    assert L.tact_compress(ctypes.byref(p), 2, kv, 32768, ctypes.c_void_p((1 << 30) + 1024),
                           wsp, ws, None) == 1
    assert L.tact_decompress(ctypes.byref(p), 2, rec, kv, 32768,
                             ctypes.c_void_p((2 << 30) + 256), ws, None) == 1
    assert L.tact_compress(None, 2, kv, 32768, rec, wsp, ws, None) == 1


def test_stage_quantizers_refuse_the_rotation():
    # the stage entry points quantize and dequantize without the rotation
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 30)
    L = lib()
    p = _params()
    assert L.tact_dbg_quantize(ctypes.byref(p), 1, fake, fake, fake, ws, 1 << 40, None) == 2
    assert L.tact_dbg_dequantize(ctypes.byref(p), 1, fake, fake, ws, 1 << 40, None) == 2
    assert b"rotation" in L.tact_last_error()


def test_stage_workspace_is_checked_first():
    fake = ctypes.c_void_p(1 << 20)
    L = lib()
    p = _params(rotation=0)
    need = L.tact_dbg_workspace_bytes(ctypes.byref(p), 2)
    # tables, then per unit the volume, variances, 1/gain, first planes, the
    # allocation's scratch, a record
    assert need >= 2 * (4 * 4 * 8 * 8 * 2 * 64)
    assert L.tact_dbg_workspace_bytes(ctypes.byref(p), 0) == 0
    assert L.tact_dbg_workspace_bytes(ctypes.byref(p), 65536) == 0
    ws = ctypes.c_void_p(1 << 30)
    for call in (lambda w, n: L.tact_dbg_dct3(ctypes.byref(p), 2, 0, fake, fake, w, n, None),
                 lambda w, n: L.tact_dbg_bin_variance(ctypes.byref(p), 2, fake, fake, w, n, None),
                 lambda w, n: L.tact_dbg_allocate(ctypes.byref(p), 2, fake, fake, w, n, None),
                 lambda w, n: L.tact_dbg_quantize(ctypes.byref(p), 2, fake, fake, fake, w, n, None),
                 lambda w, n: L.tact_dbg_dequantize(ctypes.byref(p), 2, fake, fake, w, n, None)):
        assert call(None, need) == 3
        assert call(ws, need - 1) == 3
        assert call(ctypes.c_void_p((1 << 30) + 16), need) == 1      # not 256-byte aligned
    assert L.tact_dbg_dct3(ctypes.byref(p), 65536, 0, fake, fake, ws, 1 << 45, None) == 1
    assert L.tact_dbg_allocate(ctypes.byref(p), 65536, fake, fake, ws, 1 << 45, None) == 1


def test_zero_units_is_a_noop():
    p = _params()
    assert lib().tact_compress(ctypes.byref(p), 0, None, 0, None, None, 0, None) == 0
    assert lib().tact_decompress(ctypes.byref(p), 0, None, None, 0, None, 0, None) == 0


def test_status_strings():
    for s in range(5):
        assert len(lib().tact_status_string(s)) > 0


def test_library_quantizer_tables_equal_oracle_tables():
    from oracle import QUANTIZERS, codebook_f32
    for q, name in enumerate(QUANTIZERS):
        for b in range(1, 9):
            lv, th = tact.quantizer_table(q, b)
            olv, oth = codebook_f32(b, name)
            assert torch.equal(lv, torch.from_numpy(olv)) and torch.equal(th, torch.from_numpy(oth))
    assert lib().tact_quantizer_table(3, 2, None, None) == 0
    assert lib().tact_quantizer_table(1, 0, None, None) == 0


def test_quantizer_parameter():
    p = _params()
    assert p.quantizer == 0
    for bad in (-1, 3):
        assert lib().tact_record_bytes(ctypes.byref(_params(quantizer=bad))) == 0
    fake = ctypes.c_void_p(1 << 20)
    L = lib()
    q1 = _params(quantizer=1, rotation=0)
    ws = ctypes.c_void_p(1 << 30)
    # the coding kernel of the fused layout holds the Lloyd-Max table
    assert L.tact_dbg_quantize(ctypes.byref(q1), 1, fake, fake, fake, ws, 1 << 40, None) == 2


def test_library_codebook_equals_oracle_table():
    from oracle import codebook_f32
    for b in range(1, 9):
        lv, th = tact.codebook(b)
        olv, oth = codebook_f32(b)
        assert torch.equal(lv, torch.from_numpy(olv)) and torch.equal(th, torch.from_numpy(oth))
    assert lib().tact_codebook(0, None, None) == 0
    assert lib().tact_codebook(9, None, None) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful without a GPU")
def test_valid_call_without_device_reports_hip_error():
    p = _params()
    ws = lib().tact_workspace_bytes(ctypes.byref(p), 1)
    kv, rec, wsp = (ctypes.c_void_p(a << 30) for a in (1, 2, 3))   # disjoint fake buffers
    st = lib().tact_compress(ctypes.byref(p), 1, kv, 32768, rec, wsp, ws, None)
    assert st == 4
    assert b"tact_compress" in lib().tact_last_error()


def test_attend_validation():
    L = lib()
    p = _params()                      # 4x8x8, 2 kv heads of 64
    fake = ctypes.c_void_p(1 << 20)
    ws = L.tact_attend_workspace_bytes(ctypes.byref(p), 3, 4)
    assert ws > 0
    # q_heads: a multiple of kv_heads, at most 16 per kv head
    assert L.tact_attend_workspace_bytes(ctypes.byref(p), 3, 3) == 0
    assert L.tact_attend_workspace_bytes(ctypes.byref(p), 3, 34) == 0
    assert L.tact_attend(ctypes.byref(p), 3, 3, fake, fake, fake, 1.0, fake, fake, fake, ws,
                         None) == 2
    assert L.tact_attend(ctypes.byref(p), 3, 34, fake, fake, fake, 1.0, fake, fake, fake, ws,
                         None) == 2
    # the field of S*H*W tokens must fit in LDS
    big = _params(S=64, H=32, W=32)
    assert L.tact_attend_workspace_bytes(ctypes.byref(big), 1, 2) == 0
    assert b"S*H*W" in (L.tact_attend(ctypes.byref(big), 1, 2, fake, fake, fake, 1.0, fake,
                                      fake, fake, 1 << 30, None) == 2 and L.tact_last_error())
    # pointers, alignment, scale, workspace, overlap, pair count
    args = [fake, fake, fake, 1.0, ctypes.c_void_p((1 << 20) + 65536),
            ctypes.c_void_p((1 << 20) + 131072), fake, ws]
    assert L.tact_attend(ctypes.byref(p), 3, 4, None, *args[1:], None) == 1
    assert L.tact_attend(ctypes.byref(p), 3, 4, ctypes.c_void_p((1 << 20) + 16), *args[1:],
                         None) == 1
    assert L.tact_attend(ctypes.byref(p), 3, 4, *args[:3], float("nan"), *args[4:], None) == 1
    assert L.tact_attend(ctypes.byref(p), 3, 4, *args[:6], None, ws, None) == 3
    assert L.tact_attend(ctypes.byref(p), 3, 4, *args[:7], ws - 1, None) == 3
    assert L.tact_attend(ctypes.byref(p), 3, 4, *args[:3], 1.0, fake, args[5], fake, ws,
                         None) == 1     # out overlaps q
    assert L.tact_attend(ctypes.byref(p), -1, 4, *args, None) == 1
    assert L.tact_attend(ctypes.byref(p), 0, 4, None, None, None, 1.0, None, None, None, 0,
                         None) == 0


def test_binding_rejects_mismatched_tensors_before_any_launch():
    # the checks run on the host before the library is called, so CPU
    # tensors stand in for device ones here
    g = tact.Geometry(4, 8, 8, 2, 64, 1, max_bits=3, dtype=torch.float32)
    rb = g.record_bytes()
    rec = torch.zeros((2, rb), dtype=torch.uint8)
    with pytest.raises(TypeError, match="dtype"):
        tact.decompress(rec, g, out=torch.empty((2,) + g.unit_shape, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="units"):
        tact.decompress(rec, g, out=torch.empty((1,) + g.unit_shape, dtype=torch.float32))
    with pytest.raises(ValueError, match="uint8"):
        tact.decompress(rec[:, :-1], g)
    with pytest.raises(ValueError, match="uint8"):
        tact.decompress(rec.view(torch.int8), g)
    with pytest.raises(ValueError, match="contiguous"):
        tact.decompress(torch.zeros((2, 2 * rb), dtype=torch.uint8)[:, ::2], g)
    kv = torch.zeros((2,) + g.unit_shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="records"):
        tact.compress(kv, 1, 3, records=torch.zeros((1, rb), dtype=torch.uint8))
    with pytest.raises(TypeError, match="dtype"):
        tact.roundtrip(kv, 1, 3, out=torch.empty((2,) + g.unit_shape, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        tact.compress(kv, 1, 3)
