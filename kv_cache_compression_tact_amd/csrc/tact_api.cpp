// C-ABI host layer of the TACT-KV codec: argument validation, record and
// workspace layout, chunking of large batches, launch sequencing and status
// reporting.  All compute runs in the kernels of tact_kernels.hip; this file
// never touches cache data.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "tact.h"
#include "tact_debug.h"
#include "tact_internal.h"

namespace tact {
namespace {

thread_local std::string g_last_error;

tact_status fail(tact_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

tact_status ok() {
  g_last_error.clear();
  return TACT_OK;
}

// Upper bound on the workspace one chunk of units may use; batches larger
// than a chunk are processed chunk by chunk on the same stream.
constexpr int64_t kChunkWorkspaceBytes = int64_t(2) << 30;

tact_status make_geometry(const tact_params* p, Geometry* g) {
  if (!p) return fail(TACT_ERR_INVALID_ARGUMENT, "params is NULL");
  auto in = [](int v, int lo, int hi) { return v >= lo && v <= hi; };
  if (!in(p->S, 1, 64) || !in(p->H, 1, 64) || !in(p->W, 1, 64))
    return fail(TACT_ERR_UNSUPPORTED, "grid S=%d H=%d W=%d: each must be in 1..64", p->S,
                p->H, p->W);
  if (!in(p->kv_heads, 1, 64))
    return fail(TACT_ERR_UNSUPPORTED, "kv_heads=%d: must be in 1..64", p->kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(TACT_ERR_UNSUPPORTED, "head_dim=%d: must be 64, 128 or 256", p->head_dim);
  if (!in(p->max_bits, 1, 8))
    return fail(TACT_ERR_INVALID_ARGUMENT, "max_bits=%d: must be in 1..8", p->max_bits);
  if (!in(p->budget_bits, 0, p->max_bits))
    return fail(TACT_ERR_INVALID_ARGUMENT, "budget_bits=%d: must be in 0..max_bits (%d)",
                p->budget_bits, p->max_bits);
  if (p->dtype != TACT_BF16 && p->dtype != TACT_F32)
    return fail(TACT_ERR_INVALID_ARGUMENT, "dtype=%d: must be TACT_BF16 or TACT_F32", p->dtype);
  if (!in(p->axes, 1, 7))
    return fail(TACT_ERR_INVALID_ARGUMENT, "axes=%d: must be a non-empty subset of S|H|W",
                p->axes);
  if (p->alloc_mode != TACT_ALLOC_WATERFILL && p->alloc_mode != TACT_ALLOC_UNIFORM)
    return fail(TACT_ERR_INVALID_ARGUMENT, "alloc_mode=%d: must be 0 or 1", p->alloc_mode);
  Geometry& G = *g;
  G.S = p->S;
  G.H = p->H;
  G.W = p->W;
  G.kv_heads = p->kv_heads;
  G.head_dim = p->head_dim;
  G.max_bits = p->max_bits;
  G.budget_bits = p->budget_bits;
  G.axes = p->axes;
  G.alloc_mode = p->alloc_mode;
  G.dtype = p->dtype;
  G.n_bins = int64_t(p->S) * p->H * p->W * p->kv_heads;
  G.n_entries = G.n_bins * p->head_dim;
  G.total_bits = int64_t(p->budget_bits) * G.n_bins;
  G.n_groups = (G.n_bins + 63) / 64;
  G.code_bytes = G.total_bits * p->head_dim / 8;
  G.off_gains = 0;
  G.off_bits = G.off_gains + align256(4 * G.n_bins);
  G.off_groups = G.off_bits + align256(G.n_bins);
  G.off_codes = G.off_groups + align256(4 * G.n_groups);
  G.record_bytes = G.off_codes + align256(G.code_bytes);
  return TACT_OK;
}

int64_t elem_size(int dtype) { return dtype == TACT_F32 ? 4 : 2; }

// Per-unit workspace of the codec calls: fp32 coefficients, fp32
// variances, one record.
int64_t unit_ws_bytes(const Geometry& g) {
  return align256(4 * g.n_entries) + align256(4 * g.n_bins) + g.record_bytes;
}

int64_t chunk_units(const Geometry& g, int64_t n_units) {
  int64_t c = kChunkWorkspaceBytes / unit_ws_bytes(g);
  if (c < 1) c = 1;
  if (c > 65535) c = 65535;  // grid.y limit of the transform kernels
  return n_units < c ? n_units : c;
}

struct Workspace {
  float* coef;
  float* var;
  uint8_t* recs;
};

Workspace carve(const Geometry& g, int64_t chunk, void* ws) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  Workspace w;
  w.coef = reinterpret_cast<float*>(b);
  b += chunk * align256(4 * g.n_entries);
  w.var = reinterpret_cast<float*>(b);
  b += chunk * align256(4 * g.n_bins);
  w.recs = b;
  return w;
}

bool aligned(const void* ptr, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0;
}

tact_status check_units(int64_t n_units) {
  if (n_units < 0) return fail(TACT_ERR_INVALID_ARGUMENT, "n_units=%lld < 0", (long long)n_units);
  if (n_units > (int64_t(1) << 31))
    return fail(TACT_ERR_INVALID_ARGUMENT, "n_units=%lld too large", (long long)n_units);
  return TACT_OK;
}

tact_status check_tensor(const Geometry& g, const void* ptr, int64_t stride, const char* name) {
  if (!ptr) return fail(TACT_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(ptr, 16)) return fail(TACT_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  if (stride < g.n_entries || stride % 8 != 0)
    return fail(TACT_ERR_INVALID_ARGUMENT,
                "%s unit stride %lld: must be >= %lld elements and a multiple of 8", name,
                (long long)stride, (long long)g.n_entries);
  return TACT_OK;
}

tact_status check_buffer(const void* ptr, const char* name, uintptr_t align) {
  if (!ptr) return fail(TACT_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(ptr, align))
    return fail(TACT_ERR_INVALID_ARGUMENT, "%s is not %u-byte aligned", name, (unsigned)align);
  return TACT_OK;
}

tact_status check_workspace(const Geometry& g, int64_t n_units, const void* ws, size_t bytes) {
  const int64_t need = chunk_units(g, n_units) * unit_ws_bytes(g);
  if (!ws) return fail(TACT_ERR_WORKSPACE, "workspace is NULL (%lld bytes needed)", (long long)need);
  if (!aligned(ws, 256)) return fail(TACT_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (static_cast<int64_t>(bytes) < need)
    return fail(TACT_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", bytes, (long long)need);
  return TACT_OK;
}

tact_status after_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(TACT_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  return ok();
}

RecordView view(const Geometry& g, void* base) {
  RecordView r;
  r.base = static_cast<uint8_t*>(base);
  r.stride = g.record_bytes;
  r.off_gains = g.off_gains;
  r.off_bits = g.off_bits;
  r.off_groups = g.off_groups;
  r.off_codes = g.off_codes;
  return r;
}

// compress `cn` units: kv chunk -> records chunk, workspace w
void compress_chunk(const Geometry& g, int64_t cn, const void* kv, int64_t kv_stride,
                    uint8_t* recs, const Workspace& w, hipStream_t s) {
  launch_dct3(g, cn, 0, kv, g.dtype, kv_stride, w.coef, TACT_F32, g.n_entries, nullptr, s);
  launch_bin_variance(g, cn, w.coef, w.var, s);
  launch_allocate(g, cn, w.var, nullptr, view(g, recs), s);
  launch_quantize(g, cn, w.coef, view(g, recs), s);
}

void decompress_chunk(const Geometry& g, int64_t cn, const uint8_t* recs, void* out,
                      int64_t out_stride, const Workspace& w, hipStream_t s) {
  launch_unpack(g, cn, view(g, const_cast<uint8_t*>(recs)), nullptr, w.coef, s);
  launch_dct3(g, cn, 1, w.coef, TACT_F32, g.n_entries, out, g.dtype, out_stride, w.coef, s);
}

}  // namespace
}  // namespace tact

using namespace tact;

extern "C" {

void tact_params_init(tact_params* p, int32_t S, int32_t H, int32_t W, int32_t kv_heads,
                      int32_t head_dim, int32_t budget_bits) {
  if (!p) return;
  p->S = S;
  p->H = H;
  p->W = W;
  p->kv_heads = kv_heads;
  p->head_dim = head_dim;
  p->budget_bits = budget_bits;
  p->max_bits = 8;
  p->dtype = TACT_BF16;
  p->axes = TACT_AXES_ALL;
  p->alloc_mode = TACT_ALLOC_WATERFILL;
}

size_t tact_record_bytes(const tact_params* p) {
  Geometry g;
  if (make_geometry(p, &g) != TACT_OK) return 0;
  return static_cast<size_t>(g.record_bytes);
}

size_t tact_workspace_bytes(const tact_params* p, int64_t n_units) {
  Geometry g;
  if (make_geometry(p, &g) != TACT_OK) return 0;
  if (n_units <= 0) return 0;
  return static_cast<size_t>(chunk_units(g, n_units) * unit_ws_bytes(g));
}

tact_status tact_compress(const tact_params* p, int64_t n_units, const void* kv,
                          int64_t kv_unit_stride, void* records, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_tensor(g, kv, kv_unit_stride, "kv")) != TACT_OK) return st;
  if ((st = check_buffer(records, "records", 256)) != TACT_OK) return st;
  if ((st = check_workspace(g, n_units, workspace, workspace_bytes)) != TACT_OK) return st;
  const int64_t chunk = chunk_units(g, n_units);
  const Workspace w = carve(g, chunk, workspace);
  const int64_t es = elem_size(g.dtype);
  for (int64_t u0 = 0; u0 < n_units; u0 += chunk) {
    const int64_t cn = (n_units - u0 < chunk) ? n_units - u0 : chunk;
    compress_chunk(g, cn, static_cast<const uint8_t*>(kv) + u0 * kv_unit_stride * es,
                   kv_unit_stride, static_cast<uint8_t*>(records) + u0 * g.record_bytes, w,
                   stream);
  }
  return after_launch("tact_compress");
}

tact_status tact_decompress(const tact_params* p, int64_t n_units, const void* records,
                            void* kv_out, int64_t out_unit_stride, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(records, "records", 256)) != TACT_OK) return st;
  if ((st = check_tensor(g, kv_out, out_unit_stride, "kv_out")) != TACT_OK) return st;
  if ((st = check_workspace(g, n_units, workspace, workspace_bytes)) != TACT_OK) return st;
  const int64_t chunk = chunk_units(g, n_units);
  const Workspace w = carve(g, chunk, workspace);
  const int64_t es = elem_size(g.dtype);
  for (int64_t u0 = 0; u0 < n_units; u0 += chunk) {
    const int64_t cn = (n_units - u0 < chunk) ? n_units - u0 : chunk;
    decompress_chunk(g, cn, static_cast<const uint8_t*>(records) + u0 * g.record_bytes,
                     static_cast<uint8_t*>(kv_out) + u0 * out_unit_stride * es,
                     out_unit_stride, w, stream);
  }
  return after_launch("tact_decompress");
}

tact_status tact_roundtrip(const tact_params* p, int64_t n_units, const void* kv,
                           int64_t kv_unit_stride, void* kv_out, int64_t out_unit_stride,
                           void* records, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_tensor(g, kv, kv_unit_stride, "kv")) != TACT_OK) return st;
  if ((st = check_tensor(g, kv_out, out_unit_stride, "kv_out")) != TACT_OK) return st;
  if (records && (st = check_buffer(records, "records", 256)) != TACT_OK) return st;
  if ((st = check_workspace(g, n_units, workspace, workspace_bytes)) != TACT_OK) return st;
  if (kv_out != kv && kv_unit_stride == out_unit_stride) {
    const uint8_t* a = static_cast<const uint8_t*>(kv);
    const uint8_t* b = static_cast<const uint8_t*>(kv_out);
    const int64_t span = n_units * kv_unit_stride * elem_size(g.dtype);
    if (a < b + span && b < a + span)
      return fail(TACT_ERR_INVALID_ARGUMENT, "kv and kv_out overlap without being equal");
  }
  const int64_t chunk = chunk_units(g, n_units);
  const Workspace w = carve(g, chunk, workspace);
  const int64_t es = elem_size(g.dtype);
  for (int64_t u0 = 0; u0 < n_units; u0 += chunk) {
    const int64_t cn = (n_units - u0 < chunk) ? n_units - u0 : chunk;
    uint8_t* recs = records ? static_cast<uint8_t*>(records) + u0 * g.record_bytes : w.recs;
    compress_chunk(g, cn, static_cast<const uint8_t*>(kv) + u0 * kv_unit_stride * es,
                   kv_unit_stride, recs, w, stream);
    decompress_chunk(g, cn, recs, static_cast<uint8_t*>(kv_out) + u0 * out_unit_stride * es,
                     out_unit_stride, w, stream);
  }
  return after_launch("tact_roundtrip");
}

const char* tact_status_string(tact_status s) {
  switch (s) {
    case TACT_OK: return "ok";
    case TACT_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TACT_ERR_UNSUPPORTED: return "unsupported geometry";
    case TACT_ERR_WORKSPACE: return "workspace missing or too small";
    case TACT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* tact_last_error(void) { return g_last_error.c_str(); }

int32_t tact_codebook(int32_t bits, float* levels, float* thresholds) {
  if (bits < 1 || bits > 8) return 0;
  const int n = 1 << bits;
  if (levels) std::memcpy(levels, kHostLevels + (n - 2), sizeof(float) * n);
  if (thresholds) std::memcpy(thresholds, kHostThresholds + (n - bits - 1), sizeof(float) * (n - 1));
  return n;
}

// ---------------------------------------------------------------------------
// stage entry points (tact_debug.h)
// ---------------------------------------------------------------------------
size_t tact_dbg_workspace_bytes(const tact_params* p, int64_t n_units) {
  Geometry g;
  if (make_geometry(p, &g) != TACT_OK) return 0;
  (void)n_units;
  return 0;
}

tact_status tact_dbg_dct3(const tact_params* p, int64_t n_units, int32_t inverse,
                          const void* in, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(in, "in", 16)) != TACT_OK) return st;
  if ((st = check_buffer(out, "out", 16)) != TACT_OK) return st;
  const int in_dtype = inverse ? TACT_F32 : g.dtype;
  launch_dct3(g, n_units, inverse ? 1 : 0, in, in_dtype, g.n_entries, out, TACT_F32,
              g.n_entries, nullptr, stream);
  return after_launch("tact_dbg_dct3");
}

tact_status tact_dbg_bin_variance(const tact_params* p, int64_t n_units, const float* coef,
                                  float* var, hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(coef, "coef", 16)) != TACT_OK) return st;
  if ((st = check_buffer(var, "var", 4)) != TACT_OK) return st;
  launch_bin_variance(g, n_units, coef, var, stream);
  return after_launch("tact_dbg_bin_variance");
}

tact_status tact_dbg_allocate(const tact_params* p, int64_t n_units, const float* var,
                              uint8_t* bits, hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(var, "var", 4)) != TACT_OK) return st;
  if ((st = check_buffer(bits, "bits", 1)) != TACT_OK) return st;
  RecordView none{};
  launch_allocate(g, n_units, var, bits, none, stream);
  return after_launch("tact_dbg_allocate");
}

tact_status tact_dbg_quantize(const tact_params* p, int64_t n_units, const float* coef,
                              const float* gains, const uint8_t* bits, void* records,
                              hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(coef, "coef", 16)) != TACT_OK) return st;
  if ((st = check_buffer(gains, "gains", 4)) != TACT_OK) return st;
  if ((st = check_buffer(bits, "bits", 1)) != TACT_OK) return st;
  if ((st = check_buffer(records, "records", 256)) != TACT_OK) return st;
  launch_header(g, n_units, gains, bits, view(g, records), stream);
  launch_quantize(g, n_units, coef, view(g, records), stream);
  return after_launch("tact_dbg_quantize");
}

tact_status tact_dbg_unpack(const tact_params* p, int64_t n_units, const void* records,
                            uint8_t* codes, hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(records, "records", 256)) != TACT_OK) return st;
  if ((st = check_buffer(codes, "codes", 1)) != TACT_OK) return st;
  launch_unpack(g, n_units, view(g, const_cast<void*>(records)), codes, nullptr, stream);
  return after_launch("tact_dbg_unpack");
}

tact_status tact_dbg_dequantize(const tact_params* p, int64_t n_units, const void* records,
                                float* coef, hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(records, "records", 256)) != TACT_OK) return st;
  if ((st = check_buffer(coef, "coef", 16)) != TACT_OK) return st;
  launch_unpack(g, n_units, view(g, const_cast<void*>(records)), nullptr, coef, stream);
  return after_launch("tact_dbg_dequantize");
}

}  // extern "C"
