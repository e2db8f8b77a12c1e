"""Python binding of the TACT-KV codec library (libtact.so, gfx950).

Argument marshalling only: every step of the codec runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  The
functions take and return torch tensors on the GPU:

    records = compress(kv, budget_bits)            # kv: (U, S, H, W, Hkv, d)
    kv_hat  = decompress(records, geometry...)     # bf16 / fp32 like kv
    kv_hat, records = roundtrip(kv, budget_bits)

The library is loaded from this package's directory; importing this module
without it raises ImportError (build it with
``python kv_cache_compression_tact_amd/build.py``).  There is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtact.so")

TACT_OK, TACT_ERR_INVALID_ARGUMENT, TACT_ERR_UNSUPPORTED, TACT_ERR_WORKSPACE, \
    TACT_ERR_HIP = range(5)
TACT_BF16, TACT_F32 = 0, 1
AXES_NONE, AXIS_S, AXIS_H, AXIS_W, AXES_ALL = 0, 1, 2, 4, 7
ALLOC_WATERFILL, ALLOC_UNIFORM = 0, 1
ROTATION_NONE, ROTATION_HADAMARD = 0, 1
QUANT_LLOYD_MAX, QUANT_UNIFORM, QUANT_NF = 0, 1, 2


class TactParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("S", "H", "W", "kv_heads", "head_dim", "budget_bits", "max_bits",
                 "dtype", "axes", "alloc_mode", "rotation", "quantizer")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python kv_cache_compression_tact_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(TactParams)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sigs = {
        "tact_params_init": (None, [P, i32, i32, i32, i32, i32, i32]),
        "tact_record_bytes": (sz, [P]),
        "tact_workspace_bytes": (sz, [P, i64]),
        "tact_compress": (i32, [P, i64, vp, i64, vp, vp, sz, vp]),
        "tact_decompress": (i32, [P, i64, vp, vp, i64, vp, sz, vp]),
        "tact_roundtrip": (i32, [P, i64, vp, i64, vp, i64, vp, vp, sz, vp]),
        "tact_roundtrip_noalloc": (i32, [P, i64, vp, i64, vp, i64, vp, vp]),
        "tact_status_string": (ctypes.c_char_p, [i32]),
        "tact_last_error": (ctypes.c_char_p, []),
        "tact_codebook": (i32, [i32, vp, vp]),
        "tact_quantizer_table": (i32, [i32, i32, vp, vp]),
        "tact_attend_workspace_bytes": (sz, [P, i64, i32]),
        "tact_attend": (i32, [P, i64, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]),
        "tact_dbg_workspace_bytes": (sz, [P, i64]),
        "tact_dbg_dct3": (i32, [P, i64, i32, vp, vp, vp, sz, vp]),
        "tact_dbg_bin_variance": (i32, [P, i64, vp, vp, vp, sz, vp]),
        "tact_dbg_allocate": (i32, [P, i64, vp, vp, vp, sz, vp]),
        "tact_dbg_quantize": (i32, [P, i64, vp, vp, vp, vp, sz, vp]),
        "tact_dbg_dequantize": (i32, [P, i64, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("tact_params_init", "tact_record_bytes", "tact_workspace_bytes",
            "tact_compress", "tact_decompress", "tact_roundtrip", "tact_roundtrip_noalloc",
            "tact_status_string", "tact_last_error", "tact_codebook", "tact_quantizer_table",
            "tact_attend_workspace_bytes", "tact_attend",
            "tact_dbg_workspace_bytes", "tact_dbg_dct3", "tact_dbg_bin_variance",
            "tact_dbg_allocate", "tact_dbg_quantize", "tact_dbg_dequantize")


def lib():
    """The loaded ctypes library (for tests of the raw C ABI)."""
    return _lib


class TactError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.tact_last_error().decode()
        name = _lib.tact_status_string(status).decode()
        super().__init__(f"{where}: {name} ({status}): {msg}")


def _check(status: int, where: str):
    if status != TACT_OK:
        raise TactError(status, where)


@dataclass(frozen=True)
class Geometry:
    S: int
    H: int
    W: int
    kv_heads: int
    head_dim: int
    budget_bits: int
    max_bits: int = 8
    dtype: torch.dtype = torch.bfloat16
    axes: int = AXES_ALL
    alloc_mode: int = ALLOC_WATERFILL
    rotation: int = ROTATION_HADAMARD
    quantizer: int = QUANT_LLOYD_MAX

    def params(self) -> TactParams:
        if self.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("cache dtype must be bfloat16 or float32")
        return TactParams(self.S, self.H, self.W, self.kv_heads, self.head_dim,
                          self.budget_bits, self.max_bits,
                          TACT_BF16 if self.dtype == torch.bfloat16 else TACT_F32,
                          self.axes, self.alloc_mode, self.rotation, self.quantizer)

    @property
    def unit_shape(self):
        return (self.S, self.H, self.W, self.kv_heads, self.head_dim)

    @property
    def n_bins(self) -> int:
        return self.S * self.H * self.W * self.kv_heads

    @property
    def n_entries(self) -> int:
        return self.n_bins * self.head_dim

    def record_bytes(self) -> int:
        p = self.params()
        n = _lib.tact_record_bytes(ctypes.byref(p))
        if n == 0:
            raise TactError(TACT_ERR_INVALID_ARGUMENT, "tact_record_bytes")
        return n

    def workspace_bytes(self, n_units: int) -> int:
        p = self.params()
        return _lib.tact_workspace_bytes(ctypes.byref(p), n_units)

    @staticmethod
    def of(kv: torch.Tensor, budget_bits: int, **kw) -> "Geometry":
        if kv.dim() != 6:
            raise ValueError("kv must be (units, S, H, W, kv_heads, head_dim)")
        _, S, H, W, hk, d = kv.shape
        return Geometry(S, H, W, hk, d, budget_bits, dtype=kv.dtype, **kw)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _unit_stride(t: torch.Tensor) -> int:
    """Elements between consecutive units; each unit must be contiguous."""
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if t.dim() != 6:
        raise ValueError("expected a (units, S, H, W, kv_heads, head_dim) tensor")
    unit = 1
    for n in t.shape[1:]:
        unit *= n
    if t.shape[0] == 0:
        return unit
    if not t[0].is_contiguous():
        raise ValueError("each unit must be a contiguous (S, H, W, kv_heads, head_dim) tensor")
    return t.stride(0) if t.shape[0] > 1 else unit


def _check_cache(t: torch.Tensor, geom: Geometry, n_units: int, name: str):
    """A cache tensor of the call: on the GPU, of the geometry's dtype and
    unit shape, with at least n_units units."""
    if t.dtype != geom.dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, the geometry's is {geom.dtype}")
    if t.dim() != 6 or tuple(t.shape[1:]) != geom.unit_shape:
        raise ValueError(f"{name} must be (units,) + {geom.unit_shape}, got {tuple(t.shape)}")
    if t.shape[0] < n_units:
        raise ValueError(f"{name} holds {t.shape[0]} units, the call covers {n_units}")


def _check_records(r: torch.Tensor, geom: Geometry, n_units: int, name: str = "records"):
    """Records of the call: contiguous uint8 (units, record_bytes) on the GPU,
    at least n_units rows (the library reads and writes them back to back)."""
    rb = geom.record_bytes()
    if r.dtype != torch.uint8 or r.dim() != 2 or r.shape[1] != rb:
        raise ValueError(f"{name} must be uint8 (units, {rb}), got {r.dtype} {tuple(r.shape)}")
    if r.shape[0] < n_units:
        raise ValueError(f"{name} holds {r.shape[0]} records, the call covers {n_units}")
    if not r.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    """Every tensor the call passes to the library lives on the GPU (checked
    after the shapes and types, so those errors come first)."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")


def _check_ws(ws: torch.Tensor):
    if not ws.is_cuda or ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("the workspace must be a contiguous uint8 tensor on the GPU")


def workspace(geom: Geometry, n_units: int, device=None) -> torch.Tensor:
    n = geom.workspace_bytes(n_units)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")


def compress(kv: torch.Tensor, budget_bits: int, max_bits: int = 8, *,
             records: torch.Tensor | None = None, ws: torch.Tensor | None = None,
             axes: int = AXES_ALL, alloc_mode: int = ALLOC_WATERFILL,
             rotation: int = ROTATION_HADAMARD,
             quantizer: int = QUANT_LLOYD_MAX) -> torch.Tensor:
    """kv (U, S, H, W, Hkv, d) bf16/fp32 on the GPU -> records uint8 (U, record_bytes)."""
    g = Geometry.of(kv, budget_bits, max_bits=max_bits, axes=axes, alloc_mode=alloc_mode,
                    rotation=rotation, quantizer=quantizer)
    U = kv.shape[0]
    _check_cache(kv, g, U, "kv")
    if records is None:
        records = torch.empty((U, g.record_bytes()), dtype=torch.uint8, device=kv.device)
    _check_records(records, g, U)
    _on_gpu(kv=kv, records=records)
    if ws is None:
        ws = workspace(g, U, kv.device)
    _check_ws(ws)
    p = g.params()
    _check(_lib.tact_compress(ctypes.byref(p), U, _ptr(kv), _unit_stride(kv),
                              _ptr(records), _ptr(ws), ws.numel(), _stream()),
           "tact_compress")
    return records


def decompress(records: torch.Tensor, geom: Geometry, *, out: torch.Tensor | None = None,
               ws: torch.Tensor | None = None) -> torch.Tensor:
    """records uint8 (U, record_bytes) -> cache (U, S, H, W, Hkv, d) of geom.dtype."""
    U = records.shape[0]
    _check_records(records, geom, U)
    if out is None:
        out = torch.empty((U,) + geom.unit_shape, dtype=geom.dtype, device=records.device)
    _check_cache(out, geom, U, "out")
    _on_gpu(records=records, out=out)
    if ws is None:
        ws = workspace(geom, U, records.device)
    _check_ws(ws)
    p = geom.params()
    _check(_lib.tact_decompress(ctypes.byref(p), U, _ptr(records), _ptr(out),
                                _unit_stride(out), _ptr(ws), ws.numel(), _stream()),
           "tact_decompress")
    return out


def roundtrip(kv: torch.Tensor, budget_bits: int, max_bits: int = 8, *,
              out: torch.Tensor | None = None, records: torch.Tensor | None = None,
              ws: torch.Tensor | None = None, keep_records: bool = True,
              axes: int = AXES_ALL, alloc_mode: int = ALLOC_WATERFILL,
              rotation: int = ROTATION_HADAMARD, quantizer: int = QUANT_LLOYD_MAX):
    """Compress then decompress; returns (kv_hat, records or None)."""
    g = Geometry.of(kv, budget_bits, max_bits=max_bits, axes=axes, alloc_mode=alloc_mode,
                    rotation=rotation, quantizer=quantizer)
    U = kv.shape[0]
    _check_cache(kv, g, U, "kv")
    if out is None:
        out = torch.empty_like(kv)
    _check_cache(out, g, U, "out")
    if records is None and keep_records:
        records = torch.empty((U, g.record_bytes()), dtype=torch.uint8, device=kv.device)
    if records is not None:
        _check_records(records, g, U)
    _on_gpu(kv=kv, out=out, records=records)
    if ws is None:
        ws = workspace(g, U, kv.device)
    _check_ws(ws)
    p = g.params()
    _check(_lib.tact_roundtrip(ctypes.byref(p), U, _ptr(kv), _unit_stride(kv), _ptr(out),
                               _unit_stride(out), _ptr(records), _ptr(ws), ws.numel(),
                               _stream()), "tact_roundtrip")
    return out, records


def roundtrip_noalloc(kv: torch.Tensor, budget_bits: int, max_bits: int = 8, *,
                      out: torch.Tensor, records: torch.Tensor | None = None,
                      axes: int = AXES_ALL, alloc_mode: int = ALLOC_WATERFILL,
                      rotation: int = ROTATION_HADAMARD, quantizer: int = QUANT_LLOYD_MAX):
    """roundtrip without any device allocation: the caller passes `out` (and
    `records`, or None to keep them in the library's static workspace), and
    the library's own per-GPU workspace serves the call.  Returns (out,
    records)."""
    g = Geometry.of(kv, budget_bits, max_bits=max_bits, axes=axes, alloc_mode=alloc_mode,
                    rotation=rotation, quantizer=quantizer)
    U = kv.shape[0]
    _check_cache(kv, g, U, "kv")
    _check_cache(out, g, U, "out")
    if records is not None:
        _check_records(records, g, U)
    _on_gpu(kv=kv, out=out, records=records)
    p = g.params()
    _check(_lib.tact_roundtrip_noalloc(ctypes.byref(p), U, _ptr(kv), _unit_stride(kv), _ptr(out),
                                       _unit_stride(out), _ptr(records), _stream()),
           "tact_roundtrip_noalloc")
    return out, records


STATIC_WORKSPACE_BYTES = 192 << 20    # TACT_STATIC_WORKSPACE_BYTES of tact.h


def attend_workspace(geom: Geometry, n_pairs: int, q_heads: int, device=None) -> torch.Tensor:
    p = geom.params()
    n = _lib.tact_attend_workspace_bytes(ctypes.byref(p), n_pairs, q_heads)
    if n == 0:
        _check(_lib.tact_attend(ctypes.byref(p), n_pairs, q_heads, None, None, None, 0.0, None,
                                None, None, 0, None), "tact_attend_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def attend(k_records: torch.Tensor, v_records: torch.Tensor, geom: Geometry,
           q: torch.Tensor, scale: float | None = None, *, ws: torch.Tensor | None = None):
    """One decoding step of attention over the visual tokens of unit pairs,
    read straight from the K and V records (decoding fused into attention).

    k_records, v_records: uint8 (P, record_bytes) coded with geom; q: float32
    (P, q_heads, head_dim).  Returns (out, lse): out float32 (P, q_heads,
    head_dim), the softmax-weighted sum of the decoded V over the S*H*W
    tokens; lse float32 (P, q_heads), the log-sum-exp of the scaled scores.
    """
    P, qh, d = q.shape
    if d != geom.head_dim or k_records.shape[0] != P or v_records.shape[0] != P:
        raise ValueError("q must be (pairs, q_heads, head_dim) with one K and V record per pair")
    if q.dtype != torch.float32 or not q.is_contiguous() or not q.is_cuda:
        raise TypeError("q must be contiguous float32 on the GPU")
    _check_records(k_records, geom, P, "k_records")
    _check_records(v_records, geom, P, "v_records")
    _on_gpu(k_records=k_records, v_records=v_records)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    p = geom.params()
    out = torch.empty_like(q)
    lse = torch.empty((P, qh), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = attend_workspace(geom, P, qh, q.device)
    _check_ws(ws)
    _check(_lib.tact_attend(ctypes.byref(p), P, qh, _ptr(k_records), _ptr(v_records), _ptr(q),
                            float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream()),
           "tact_attend")
    return out, lse


def quantizer_table(quantizer: int, bits: int):
    """The library's fp32 table of any quantizer (levels, thresholds), CPU tensors."""
    n = 1 << bits
    lv = torch.empty(n, dtype=torch.float32)
    th = torch.empty(n - 1, dtype=torch.float32)
    if _lib.tact_quantizer_table(quantizer, bits, lv.data_ptr(), th.data_ptr()) != n:
        raise ValueError(f"invalid quantizer {quantizer} or bit width {bits}")
    return lv, th


def codebook(bits: int):
    """The library's fp32 Lloyd-Max table (levels, thresholds) as CPU tensors."""
    n = 1 << bits
    lv = torch.empty(n, dtype=torch.float32)
    th = torch.empty(n - 1, dtype=torch.float32)
    got = _lib.tact_codebook(bits, _ptr(lv), _ptr(th))
    if got != n:
        raise ValueError("bits must be in 1..8")
    return lv, th


# ---- stage entry points ----------------------------------------------------
# Each runs the codec's own kernels up to (or from) one step of the method;
# the tensors are packed units on the GPU.
def _dbg_ws(geom: Geometry, n_units: int, device) -> torch.Tensor:
    p = geom.params()
    n = _lib.tact_dbg_workspace_bytes(ctypes.byref(p), n_units)
    if n == 0:
        raise ValueError(f"no stage workspace for {n_units} units of {geom}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _check_packed(t: torch.Tensor, shape, dtype, name: str):
    if not t.is_cuda or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def dbg_dct3(x: torch.Tensor, geom: Geometry, inverse: bool = False) -> torch.Tensor:
    """Forward: the fp32 coefficients of the cache tensors x (the geometry's
    dtype) as the coding passes compute them, without the rotation.
    Inverse: the fp32 inverse transform of fp32 coefficients x."""
    U = x.shape[0]
    _check_packed(x, (U,) + geom.unit_shape, torch.float32 if inverse else geom.dtype, "x")
    out = torch.empty((U,) + geom.unit_shape, dtype=torch.float32, device=x.device)
    if U == 0:
        return out
    p = geom.params()
    ws = _dbg_ws(geom, U, x.device)
    _check(_lib.tact_dbg_dct3(ctypes.byref(p), U, 1 if inverse else 0, _ptr(x), _ptr(out),
                              _ptr(ws), ws.numel(), _stream()), "tact_dbg_dct3")
    return out


def dbg_bin_variance(x: torch.Tensor, geom: Geometry) -> torch.Tensor:
    """Per-bin variances of the cache tensors x, as the allocation reads them."""
    U = x.shape[0]
    _check_packed(x, (U,) + geom.unit_shape, geom.dtype, "x")
    var = torch.empty((U,) + geom.unit_shape[:-1], dtype=torch.float32, device=x.device)
    if U == 0:
        return var
    p = geom.params()
    ws = _dbg_ws(geom, U, x.device)
    _check(_lib.tact_dbg_bin_variance(ctypes.byref(p), U, _ptr(x), _ptr(var), _ptr(ws),
                                      ws.numel(), _stream()), "tact_dbg_bin_variance")
    return var


def dbg_allocate(var: torch.Tensor, geom: Geometry) -> torch.Tensor:
    """Bit widths of every bin from fp32 variances (units, S, H, W, kv_heads)."""
    U = var.shape[0]
    _check_packed(var, (U,) + geom.unit_shape[:-1], torch.float32, "var")
    bits = torch.empty((U,) + geom.unit_shape[:-1], dtype=torch.uint8, device=var.device)
    if U == 0:
        return bits
    p = geom.params()
    ws = _dbg_ws(geom, U, var.device)
    _check(_lib.tact_dbg_allocate(ctypes.byref(p), U, _ptr(var), _ptr(bits), _ptr(ws), ws.numel(),
                                  _stream()), "tact_dbg_allocate")
    return bits


def dbg_quantize(coef: torch.Tensor, var: torch.Tensor, geom: Geometry) -> torch.Tensor:
    """Records of fp32 coefficients, coded as given, with the allocation of
    fp32 variances var (units, S, H, W, kv_heads)."""
    U = coef.shape[0]
    _check_packed(coef, (U,) + geom.unit_shape, torch.float32, "coef")
    _check_packed(var, (U,) + geom.unit_shape[:-1], torch.float32, "var")
    rec = torch.empty((U, geom.record_bytes()), dtype=torch.uint8, device=coef.device)
    if U == 0:
        return rec
    p = geom.params()
    ws = _dbg_ws(geom, U, coef.device)
    _check(_lib.tact_dbg_quantize(ctypes.byref(p), U, _ptr(coef), _ptr(var), _ptr(rec),
                                  _ptr(ws), ws.numel(), _stream()), "tact_dbg_quantize")
    return rec


def dbg_dequantize(records: torch.Tensor, geom: Geometry) -> torch.Tensor:
    """fp32 g * level[code] of every coefficient of the records, by the first
    decoding kernel (identity matrices in place of the DCT)."""
    U = records.shape[0]
    _check_packed(records, (U, geom.record_bytes()), torch.uint8, "records")
    coef = torch.empty((U,) + geom.unit_shape, dtype=torch.float32, device=records.device)
    if U == 0:
        return coef
    p = geom.params()
    ws = _dbg_ws(geom, U, records.device)
    _check(_lib.tact_dbg_dequantize(ctypes.byref(p), U, _ptr(records), _ptr(coef), _ptr(ws),
                                    ws.numel(), _stream()), "tact_dbg_dequantize")
    return coef
