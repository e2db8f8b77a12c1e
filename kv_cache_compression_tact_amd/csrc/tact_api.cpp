// C-ABI host layer of the TACT-KV codec: argument validation, record and
// workspace layout, chunking of large batches, launch sequencing and status
// reporting.  All compute runs in the kernels of tact_kernels.hip; this file
// never touches cache data.
#include <cmath>
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

int64_t elem_size(int dtype) { return dtype == TACT_F32 ? 4 : 2; }

// Units of one chunk are at most this many (the kernels index units of a
// launch in 16 bits of the grid).  Batches are processed chunk by chunk on
// the same stream; the chunk is as many units as the caller's workspace
// holds, so tact_workspace_bytes(p, n) (room for all n units) runs every
// kernel once over the whole batch, and any smaller workspace that holds one
// unit is accepted.
constexpr int64_t kMaxChunkUnits = 65535;

// rows of the matrix tile an axis of length n is padded to
int64_t padded_axis(int n) { return n <= 16 ? 16 : n <= 32 ? 32 : 64; }
// fp32 bytes of a unit with every grid axis padded to its tile
int64_t padded_unit_bytes(const Geometry& g) {
  return 4 * padded_axis(g.S) * padded_axis(g.H) * padded_axis(g.W) *
         static_cast<int64_t>(g.kv_heads) * g.head_dim;
}
constexpr int64_t kMaxPaddedUnitBytes = int64_t(1) << 30;

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
  if (!in(p->axes, 0, 7))
    return fail(TACT_ERR_INVALID_ARGUMENT, "axes=%d: must be a subset of S|H|W", p->axes);
  if (p->alloc_mode != TACT_ALLOC_WATERFILL && p->alloc_mode != TACT_ALLOC_UNIFORM)
    return fail(TACT_ERR_INVALID_ARGUMENT, "alloc_mode=%d: must be 0 or 1", p->alloc_mode);
  if (p->rotation != TACT_ROTATION_NONE && p->rotation != TACT_ROTATION_HADAMARD)
    return fail(TACT_ERR_INVALID_ARGUMENT, "rotation=%d: must be 0 or 1", p->rotation);
  if (p->quantizer < TACT_QUANT_LLOYD_MAX || p->quantizer > TACT_QUANT_NF)
    return fail(TACT_ERR_INVALID_ARGUMENT, "quantizer=%d: must be 0, 1 or 2", p->quantizer);
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
  G.rotation = p->rotation;
  G.quantizer = p->quantizer;
  G.dtype = p->dtype;
  G.n_bins = int64_t(p->S) * p->H * p->W * p->kv_heads;
  G.n_entries = G.n_bins * p->head_dim;
  // The kernels address a unit's fp32 volume through buffer descriptors with
  // 32-bit offsets, rows of an axis padded to the 16, 32 or 64 rows of its
  // matrix tile, and send dropped lanes to an offset just under 2^31.  With
  // the padded volume at most 2^30 bytes, every offset a kernel forms (a
  // padded row plus a column, below twice that) stays under 2^31, every
  // descriptor range stays under the dropped offset, and no sum of offsets
  // wraps past 2^32 into a range.
  if (padded_unit_bytes(G) > kMaxPaddedUnitBytes)
    return fail(TACT_ERR_UNSUPPORTED,
                "unit S=%d H=%d W=%d x %d x %d: padded fp32 volume of %lld bytes, at most 2^30",
                p->S, p->H, p->W, p->kv_heads, p->head_dim,
                static_cast<long long>(padded_unit_bytes(G)));
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


// Workspace of the codec calls: DCT tables once, then per unit of a chunk an
// fp32 intermediate volume, fp32 variances, fp32 reciprocal gains, uint32
// per-bin first planes and one record (used by tact_roundtrip when
// records == NULL).
// per-bin partial sums of squares: one per 64-channel slab of a head
int64_t var_parts(const Geometry& g) { return g.head_dim / 64; }

// floats between the variances (and reciprocal gains) of consecutive units
int64_t var_stride(const Geometry& g) { return align256(4 * g.n_bins * var_parts(g)) / 4; }

int64_t unit_ws_bytes(const Geometry& g) {
  return align256(4 * g.n_entries) + 4 * 2 * var_stride(g) + align256(4 * g.n_bins) +
         kAllocScratchBytes + g.record_bytes;
}

constexpr int64_t kTableBytes = align256(4 * kDctTableFloats);

// Workspace for a chunk of `chunk` units.
int64_t ws_bytes(const Geometry& g, int64_t chunk) {
  return kTableBytes + chunk * unit_ws_bytes(g);
}

// Units per chunk that a workspace of `bytes` bytes holds (at least 1: the
// caller has checked that one unit fits), at most n_units.
int64_t chunk_units(const Geometry& g, int64_t n_units, size_t bytes) {
  int64_t c = (static_cast<int64_t>(bytes) - kTableBytes) / unit_ws_bytes(g);
  if (c < 1) c = 1;
  if (c > kMaxChunkUnits) c = kMaxChunkUnits;
  return n_units < c ? n_units : c;
}

struct Workspace {
  float* tab;
  float* coef;
  float* var;
  float* invg;
  uint32_t* poff;
  uint8_t* alloc;      // the allocation's scratch
  uint8_t* recs;
};

Workspace carve(const Geometry& g, int64_t chunk, void* ws) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  Workspace w;
  w.tab = reinterpret_cast<float*>(b);
  b += kTableBytes;
  w.coef = reinterpret_cast<float*>(b);
  b += chunk * align256(4 * g.n_entries);
  w.var = reinterpret_cast<float*>(b);
  b += chunk * 4 * var_stride(g);
  w.invg = reinterpret_cast<float*>(b);
  b += chunk * 4 * var_stride(g);
  w.poff = reinterpret_cast<uint32_t*>(b);
  b += chunk * align256(4 * g.n_bins);
  w.alloc = b;
  b += chunk * kAllocScratchBytes;
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

// The workspace must hold one unit; a larger one lets more units share each
// launch (see chunk_units).
tact_status check_workspace(const Geometry& g, const void* ws, size_t bytes) {
  const int64_t need = ws_bytes(g, 1);
  if (!ws) return fail(TACT_ERR_WORKSPACE, "workspace is NULL (%lld bytes needed)", (long long)need);
  if (!aligned(ws, 256)) return fail(TACT_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (static_cast<int64_t>(bytes) < need)
    return fail(TACT_ERR_WORKSPACE, "workspace of %zu bytes, at least %lld needed (one unit)",
                bytes, (long long)need);
  return TACT_OK;
}

// Byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uint8_t* x = static_cast<const uint8_t*>(a);
  const uint8_t* y = static_cast<const uint8_t*>(b);
  return x < y + nb && y < x + na;
}

// Bytes spanned by n_units unit tensors `stride` elements apart.
int64_t tensor_span(const Geometry& g, int64_t n_units, int64_t stride) {
  return ((n_units - 1) * stride + g.n_entries) * elem_size(g.dtype);
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

// Transform axes in forward order (S, H, W) restricted to the mask.  With no
// axis the S pass runs with the identity matrix in place of the DCT (the
// tables kernel writes it for axes == 0), so coding needs no separate path.
int forward_axes(const Geometry& g, int* ax) {
  int m = 0;
  for (int a = 0; a < 3; ++a)
    if (g.axes & (1 << a)) ax[m++] = a;
  if (m == 0) ax[m++] = 0;
  return m;
}

// The fused layout: S on the matrix cores into the fp32 volume, then H and W
// together in LDS (tact_mfma.hip k_plane), coding in one streaming pass
// (tact_quant.hip).  Other geometries run the axes as separate passes.
bool fused_path(const Geometry& g) {
  return g.axes == TACT_AXES_ALL && plane_supported(g) && g.quantizer == TACT_QUANT_LLOYD_MAX;
}

// Where the forward stage leaves the per-bin sums of squares.
struct StatsLayout {
  int parts;      // partial sums per bin
  bool planes;    // stored plane by plane ([slab][s][kh][kw]) rather than per bin
};

// Stage 2 and the sums of stage 3 for `cn` units.  Fused path: the S pass
// writes the fp32 volume (and applies the quantizer's rotation to its output:
// the rotation acts on the channels, so it commutes with the H and W axes and
// leaves the bin variances unchanged); the plane pass replaces the volume by
// the final coefficients and writes the partial sums.  Otherwise every axis
// but the last runs forward into the volume, and the last one runs with the
// sums-of-squares epilogue (no coefficients are written).  In both cases
// w.var then holds what the allocation reads.
StatsLayout forward_stats(const Geometry& g, int64_t cn, const void* kv, int64_t kv_stride,
                          const Workspace& w, hipStream_t s) {
  const RecordView none{};
  const int in_pro = g.dtype == TACT_BF16 ? AX_PRO_BF16 : AX_PRO_F32;
  const int64_t vs = var_stride(g);
  if (fused_path(g)) {
    launch_axis(g, cn, 0, 0, in_pro, AX_EPI_F32, kv, kv_stride, w.coef, g.n_entries, w.tab,
                nullptr, nullptr, 0, none, nullptr, s, /*rot_in=*/false, /*rot_out=*/true);
    launch_plane(g, cn, 0, w.coef, w.coef, g.n_entries, w.tab, w.var, vs, none, nullptr, s);
    return {static_cast<int>(var_parts(g)), true};
  }
  int ax[3];
  const int m = forward_axes(g, ax);
  for (int j = 0; j + 1 < m; ++j) {
    if (j == 0)
      launch_axis(g, cn, ax[j], 0, in_pro, AX_EPI_F32, kv, kv_stride, w.coef, g.n_entries,
                  w.tab, nullptr, nullptr, 0, none, nullptr, s);
    else
      launch_axis(g, cn, ax[j], 0, AX_PRO_F32, AX_EPI_F32, w.coef, g.n_entries, w.coef,
                  g.n_entries, w.tab, nullptr, nullptr, 0, none, nullptr, s);
  }
  launch_axis(g, cn, ax[m - 1], 0, m == 1 ? in_pro : AX_PRO_F32, AX_EPI_STATS,
              m == 1 ? kv : static_cast<const void*>(w.coef), m == 1 ? kv_stride : g.n_entries,
              nullptr, 0, w.tab, w.var, nullptr, vs, none, nullptr, s);
  return {1, false};
}

// compress `cn` units: kv chunk -> records chunk.  The allocation reads the
// sums of the forward stage and leaves the record header, the first planes
// and the reciprocal gains; the coding pass then reads the final
// coefficients (fused path) or runs the last axis again with the coding
// epilogue.
void compress_chunk(const Geometry& g, int64_t cn, const void* kv, int64_t kv_stride,
                    uint8_t* recs, const Workspace& w, hipStream_t s) {
  const int64_t vs = var_stride(g);
  const float inv_d = 1.0f / static_cast<float>(g.head_dim);
  const StatsLayout sl = forward_stats(g, cn, kv, kv_stride, w, s);
  if (fused_path(g)) {
    // the coding pass takes first planes and 1/gain from the record header
    launch_allocate2(g, cn, w.var, vs, sl.parts, inv_d, nullptr, view(g, recs), nullptr, nullptr,
                     w.alloc, s, sl.planes);
    launch_quant(g, cn, w.coef, g.n_entries, view(g, recs), s);
    return;
  }
  launch_allocate2(g, cn, w.var, vs, sl.parts, inv_d, nullptr, view(g, recs), w.poff, w.invg,
                   w.alloc, s, sl.planes);
  int ax[3];
  const int m = forward_axes(g, ax);
  const int in_pro = g.dtype == TACT_BF16 ? AX_PRO_BF16 : AX_PRO_F32;
  launch_axis(g, cn, ax[m - 1], 0, m == 1 ? in_pro : AX_PRO_F32, AX_EPI_QUANT,
              m == 1 ? kv : static_cast<const void*>(w.coef), m == 1 ? kv_stride : g.n_entries,
              nullptr, 0, w.tab, nullptr, w.invg, vs, view(g, recs), w.poff, s);
}

// decompress `cn` records: the last forward axis runs first, reading and
// dequantizing the codes; the remaining axes run in reverse order, the last
// one writing the cache.
void decompress_chunk(const Geometry& g, int64_t cn, const uint8_t* recs, void* out,
                      int64_t out_stride, const Workspace& w, hipStream_t s) {
  const RecordView rv = view(g, const_cast<uint8_t*>(recs));
  const int out_epi = g.dtype == TACT_BF16 ? AX_EPI_BF16 : AX_EPI_F32;
  launch_plane_offsets(g, cn, rv, w.poff, s);
  if (fused_path(g)) {
    launch_plane(g, cn, 2, nullptr, w.coef, g.n_entries, w.tab, nullptr, 0, rv, w.poff, s);
    // the inverse S axis also undoes the quantizer's rotation (it acts on
    // the channels, so it commutes with the transform)
    launch_axis(g, cn, 0, 1, AX_PRO_F32, out_epi, w.coef, g.n_entries, out, out_stride, w.tab,
                nullptr, nullptr, 0, rv, w.poff, s, /*rot_in=*/true);
    return;
  }
  int ax[3];
  const int m = forward_axes(g, ax);
  for (int j = m - 1; j >= 0; --j) {
    const bool first = (j == m - 1), last = (j == 0);
    const int pro = first ? AX_PRO_DEQUANT : AX_PRO_F32;
    const int epi = last ? out_epi : AX_EPI_F32;
    void* o = last ? out : static_cast<void*>(w.coef);
    const int64_t os = last ? out_stride : g.n_entries;
    launch_axis(g, cn, ax[j], 1, pro, epi, w.coef, g.n_entries, o, os, w.tab, nullptr, nullptr, 0,
                rv, w.poff, s);
  }
}

}  // namespace
}  // namespace tact

// ---- decoding fused into attention ---------------------------------------
namespace tact {
namespace {

constexpr int64_t kMaxAttendField = 40000;   // S*H*W fp32 held in LDS (160 KB)

struct AttendWs {
  float* tab;
  uint32_t* frags;
  uint32_t* kpoff;
  uint32_t* vpoff;
  float* qrot;
  float* field;
  float* partial;
};

int64_t attend_ws_bytes(const Geometry& g, int64_t n_pairs, int q_heads, AttendWs* w,
                        void* base) {
  uint8_t* b = static_cast<uint8_t*>(base);
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    uint8_t* ptr = b ? b + off : nullptr;
    off += align256(bytes);
    return ptr;
  };
  const int64_t shw = static_cast<int64_t>(g.S) * g.H * g.W;
  const int rep = q_heads / g.kv_heads;
  AttendWs x;
  x.tab = reinterpret_cast<float*>(take(4 * kDctTableFloats));
  x.frags = reinterpret_cast<uint32_t*>(take(kAttendFragBytes));
  x.kpoff = reinterpret_cast<uint32_t*>(take(4 * n_pairs * g.n_bins));
  x.vpoff = reinterpret_cast<uint32_t*>(take(4 * n_pairs * g.n_bins));
  x.qrot = reinterpret_cast<float*>(take(4 * n_pairs * q_heads * g.head_dim));
  x.field = reinterpret_cast<float*>(take(4 * n_pairs * q_heads * shw));
  x.partial = reinterpret_cast<float*>(
      take(4 * n_pairs * g.kv_heads * attend_chunks(g) * rep * g.head_dim));
  if (w) *w = x;
  return off;
}

tact_status check_attend(const Geometry& g, int64_t n_pairs, int32_t q_heads) {
  if (n_pairs < 0 || n_pairs > 65535)
    return fail(TACT_ERR_INVALID_ARGUMENT, "n_pairs=%lld: must be in 0..65535", (long long)n_pairs);
  if (q_heads < g.kv_heads || q_heads % g.kv_heads != 0)
    return fail(TACT_ERR_UNSUPPORTED, "q_heads=%d: must be a multiple of kv_heads=%d", q_heads,
                g.kv_heads);
  if (q_heads / g.kv_heads > kMaxAttendRep)
    return fail(TACT_ERR_UNSUPPORTED, "%d query heads per kv head: at most %d",
                q_heads / g.kv_heads, kMaxAttendRep);
  if (static_cast<int64_t>(g.S) * g.H * g.W > kMaxAttendField)
    return fail(TACT_ERR_UNSUPPORTED, "S*H*W=%lld: at most %lld for attention",
                static_cast<long long>(g.S) * g.H * g.W, (long long)kMaxAttendField);
  return TACT_OK;
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
  p->rotation = TACT_ROTATION_HADAMARD;
  p->quantizer = TACT_QUANT_LLOYD_MAX;
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
  return static_cast<size_t>(ws_bytes(g, n_units < kMaxChunkUnits ? n_units : kMaxChunkUnits));
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
  if ((st = check_workspace(g, workspace, workspace_bytes)) != TACT_OK) return st;
  {
    const int64_t kv_span = tensor_span(g, n_units, kv_unit_stride);
    const int64_t rec_span = n_units * g.record_bytes;
    if (overlap(kv, kv_span, records, rec_span) ||
        overlap(kv, kv_span, workspace, static_cast<int64_t>(workspace_bytes)) ||
        overlap(records, rec_span, workspace, static_cast<int64_t>(workspace_bytes)))
      return fail(TACT_ERR_INVALID_ARGUMENT, "kv, records and workspace must not overlap");
  }
  const int64_t chunk = chunk_units(g, n_units, workspace_bytes);
  const Workspace w = carve(g, chunk, workspace);
  const int64_t es = elem_size(g.dtype);
  launch_dct_tables(g, w.tab, stream);
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
  if ((st = check_workspace(g, workspace, workspace_bytes)) != TACT_OK) return st;
  {
    const int64_t out_span = tensor_span(g, n_units, out_unit_stride);
    const int64_t rec_span = n_units * g.record_bytes;
    if (overlap(kv_out, out_span, records, rec_span) ||
        overlap(kv_out, out_span, workspace, static_cast<int64_t>(workspace_bytes)) ||
        overlap(records, rec_span, workspace, static_cast<int64_t>(workspace_bytes)))
      return fail(TACT_ERR_INVALID_ARGUMENT, "records, kv_out and workspace must not overlap");
  }
  const int64_t chunk = chunk_units(g, n_units, workspace_bytes);
  const Workspace w = carve(g, chunk, workspace);
  const int64_t es = elem_size(g.dtype);
  launch_dct_tables(g, w.tab, stream);
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
  if ((st = check_workspace(g, workspace, workspace_bytes)) != TACT_OK) return st;
  {
    // in place (kv_out == kv) only with equal strides: a chunk's output
    // must not land on input units of a later chunk
    const int64_t kv_span = tensor_span(g, n_units, kv_unit_stride);
    const int64_t out_span = tensor_span(g, n_units, out_unit_stride);
    const int64_t wsb = static_cast<int64_t>(workspace_bytes);
    if (kv_out == kv) {
      if (kv_unit_stride != out_unit_stride)
        return fail(TACT_ERR_INVALID_ARGUMENT,
                    "in-place round trip (kv_out == kv) needs equal unit strides (%lld, %lld)",
                    (long long)kv_unit_stride, (long long)out_unit_stride);
    } else if (overlap(kv, kv_span, kv_out, out_span)) {
      return fail(TACT_ERR_INVALID_ARGUMENT, "kv and kv_out overlap without being equal");
    }
    const int64_t rec_span = records ? n_units * g.record_bytes : 0;
    if (overlap(kv, kv_span, workspace, wsb) || overlap(kv_out, out_span, workspace, wsb) ||
        (records && (overlap(records, rec_span, kv, kv_span) ||
                     overlap(records, rec_span, kv_out, out_span) ||
                     overlap(records, rec_span, workspace, wsb))))
      return fail(TACT_ERR_INVALID_ARGUMENT, "kv, kv_out, records and workspace must not overlap");
  }
  const int64_t chunk = chunk_units(g, n_units, workspace_bytes);
  const Workspace w = carve(g, chunk, workspace);
  const int64_t es = elem_size(g.dtype);
  launch_dct_tables(g, w.tab, stream);
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

tact_status tact_roundtrip_noalloc(const tact_params* p, int64_t n_units, const void* kv,
                                   int64_t kv_unit_stride, void* kv_out, int64_t out_unit_stride,
                                   void* records, hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units == 0) return ok();
  const int64_t need = ws_bytes(g, 1);
  if (need > static_cast<int64_t>(TACT_STATIC_WORKSPACE_BYTES))
    return fail(TACT_ERR_UNSUPPORTED,
                "tact_roundtrip_noalloc: one unit of this geometry needs %lld bytes of "
                "workspace; the library's static workspace holds %lld (use tact_roundtrip "
                "with a caller workspace)",
                (long long)need, (long long)TACT_STATIC_WORKSPACE_BYTES);
  void* ws = nullptr;
  const hipError_t e = static_workspace(&ws);
  if (e != hipSuccess)
    return fail(TACT_ERR_HIP, "tact_roundtrip_noalloc: static workspace: %s (%s)",
                hipGetErrorName(e), hipGetErrorString(e));
  return tact_roundtrip(p, n_units, kv, kv_unit_stride, kv_out, out_unit_stride, records, ws,
                        TACT_STATIC_WORKSPACE_BYTES, stream);
}

size_t tact_attend_workspace_bytes(const tact_params* p, int64_t n_pairs, int32_t q_heads) {
  Geometry g;
  if (make_geometry(p, &g) != TACT_OK || check_attend(g, n_pairs, q_heads) != TACT_OK) return 0;
  return static_cast<size_t>(attend_ws_bytes(g, n_pairs, q_heads, nullptr, nullptr));
}

tact_status tact_attend(const tact_params* p, int64_t n_pairs, int32_t q_heads,
                        const void* k_records, const void* v_records, const float* q,
                        float scale, float* out, float* lse, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  Geometry g;
  tact_status st;
  if ((st = make_geometry(p, &g)) != TACT_OK) return st;
  if ((st = check_attend(g, n_pairs, q_heads)) != TACT_OK) return st;
  if (n_pairs == 0) return ok();
  if ((st = check_buffer(k_records, "k_records", 256)) != TACT_OK) return st;
  if ((st = check_buffer(v_records, "v_records", 256)) != TACT_OK) return st;
  if ((st = check_buffer(q, "q", 4)) != TACT_OK) return st;
  if ((st = check_buffer(out, "out", 4)) != TACT_OK) return st;
  if ((st = check_buffer(lse, "lse", 4)) != TACT_OK) return st;
  if (!std::isfinite(scale)) return fail(TACT_ERR_INVALID_ARGUMENT, "scale is not finite");
  const int64_t need = attend_ws_bytes(g, n_pairs, q_heads, nullptr, nullptr);
  if (!workspace)
    return fail(TACT_ERR_WORKSPACE, "workspace is NULL (%lld bytes needed)", (long long)need);
  if (!aligned(workspace, 256)) return fail(TACT_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (static_cast<int64_t>(workspace_bytes) < need)
    return fail(TACT_ERR_WORKSPACE, "workspace of %zu bytes, %lld needed", workspace_bytes,
                (long long)need);
  {
    // out and lse may not overlap q or each other
    const uint8_t* a0 = reinterpret_cast<const uint8_t*>(q);
    const uint8_t* b0 = reinterpret_cast<const uint8_t*>(out);
    const uint8_t* c0 = reinterpret_cast<const uint8_t*>(lse);
    const int64_t nq = 4 * n_pairs * q_heads * g.head_dim, nl = 4 * n_pairs * q_heads;
    auto over = [](const uint8_t* x, int64_t nx, const uint8_t* y, int64_t ny) {
      return x < y + ny && y < x + nx;
    };
    if (over(a0, nq, b0, nq) || over(a0, nq, c0, nl) || over(b0, nq, c0, nl))
      return fail(TACT_ERR_INVALID_ARGUMENT, "q, out and lse overlap");
  }
  AttendWs w;
  attend_ws_bytes(g, n_pairs, q_heads, &w, workspace);
  const RecordView kv = view(g, const_cast<void*>(k_records));
  const RecordView vv = view(g, const_cast<void*>(v_records));
  launch_dct_tables(g, w.tab, stream);
  launch_plane_offsets(g, n_pairs, kv, w.kpoff, stream, &vv, w.vpoff);
  launch_attend(g, n_pairs, q_heads, kv, vv, w.kpoff, w.vpoff, q, scale, w.qrot, w.field,
                w.partial, out, lse, w.tab, w.frags, stream);
  return after_launch("tact_attend");
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

int32_t tact_quantizer_table(int32_t quantizer, int32_t bits, float* levels, float* thresholds) {
  if (bits < 1 || bits > 8 || quantizer < TACT_QUANT_LLOYD_MAX || quantizer > TACT_QUANT_NF)
    return 0;
  const int n = 1 << bits;
  if (levels) std::memcpy(levels, kHostLevelsQ[quantizer] + (n - 2), sizeof(float) * n);
  if (thresholds)
    std::memcpy(thresholds, kHostThresholdsQ[quantizer] + (n - bits - 1), sizeof(float) * (n - 1));
  return n;
}

int32_t tact_codebook(int32_t bits, float* levels, float* thresholds) {
  if (bits < 1 || bits > 8) return 0;
  const int n = 1 << bits;
  if (levels) std::memcpy(levels, kHostLevels + (n - 2), sizeof(float) * n);
  if (thresholds) std::memcpy(thresholds, kHostThresholds + (n - bits - 1), sizeof(float) * (n - 1));
  return n;
}

// ---------------------------------------------------------------------------
// stage entry points (tact_debug.h): each runs the kernels tact_compress and
// tact_decompress launch, on the whole batch at once (no chunking)
// ---------------------------------------------------------------------------
size_t tact_dbg_workspace_bytes(const tact_params* p, int64_t n_units) {
  Geometry g;
  if (make_geometry(p, &g) != TACT_OK || n_units <= 0 || n_units > kMaxChunkUnits) return 0;
  return static_cast<size_t>(ws_bytes(g, n_units));
}

namespace {

// Common checks of the stage calls; on success *w is the carved workspace.
tact_status dbg_prologue(const char* who, const tact_params* p, int64_t n_units, void* ws,
                         size_t ws_bytes_given, Geometry* g, Workspace* w) {
  tact_status st;
  if ((st = make_geometry(p, g)) != TACT_OK) return st;
  if ((st = check_units(n_units)) != TACT_OK) return st;
  if (n_units > kMaxChunkUnits)
    return fail(TACT_ERR_INVALID_ARGUMENT, "%s: n_units=%lld, at most %lld per stage call", who,
                (long long)n_units, (long long)kMaxChunkUnits);
  if (n_units == 0) return TACT_OK;
  const int64_t need = ws_bytes(*g, n_units);
  if (!ws) return fail(TACT_ERR_WORKSPACE, "%s: workspace is NULL (%lld bytes needed)", who,
                       (long long)need);
  if (!aligned(ws, 256))
    return fail(TACT_ERR_INVALID_ARGUMENT, "%s: workspace is not 256-byte aligned", who);
  if (static_cast<int64_t>(ws_bytes_given) < need)
    return fail(TACT_ERR_WORKSPACE, "%s: workspace of %zu bytes, %lld needed", who,
                ws_bytes_given, (long long)need);
  *w = carve(*g, n_units, ws);
  return TACT_OK;
}

}  // namespace

tact_status tact_dbg_dct3(const tact_params* p, int64_t n_units, int32_t inverse,
                          const void* in, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  Geometry g;
  Workspace w;
  tact_status st;
  if ((st = dbg_prologue("tact_dbg_dct3", p, n_units, workspace, workspace_bytes, &g, &w)) !=
      TACT_OK)
    return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(in, "in", 16)) != TACT_OK) return st;
  if ((st = check_buffer(out, "out", 16)) != TACT_OK) return st;
  // the plain transform: the quantizer's rotation stays off
  g.rotation = TACT_ROTATION_NONE;
  launch_dct_tables(g, w.tab, stream);
  const RecordView none{};
  if (!inverse && fused_path(g)) {
    // the product's S pass, then the plane pass in place in `out`
    const int in_pro = g.dtype == TACT_BF16 ? AX_PRO_BF16 : AX_PRO_F32;
    launch_axis(g, n_units, 0, 0, in_pro, AX_EPI_F32, in, g.n_entries, out, g.n_entries, w.tab,
                nullptr, nullptr, 0, none, nullptr, stream);
    launch_plane(g, n_units, 0, out, out, g.n_entries, w.tab, w.var, var_stride(g), none,
                 nullptr, stream);
    return after_launch("tact_dbg_dct3");
  }
  // axis by axis, as the decoding of every geometry and the coding of the
  // others run them (the last forward axis of the coding pass runs there
  // with its sums-of-squares and coding epilogues instead)
  int ax[3];
  const int m = forward_axes(g, ax);
  for (int j = 0; j < m; ++j) {
    const int a = inverse ? ax[m - 1 - j] : ax[j];
    const int pro = (j == 0 && !inverse && g.dtype == TACT_BF16) ? AX_PRO_BF16 : AX_PRO_F32;
    const void* src = (j == 0) ? in : static_cast<const void*>(out);
    launch_axis(g, n_units, a, inverse ? 1 : 0, pro, AX_EPI_F32, src, g.n_entries, out,
                g.n_entries, w.tab, nullptr, nullptr, 0, none, nullptr, stream);
  }
  return after_launch("tact_dbg_dct3");
}

tact_status tact_dbg_bin_variance(const tact_params* p, int64_t n_units, const void* kv,
                                  float* var, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  Geometry g;
  Workspace w;
  tact_status st;
  if ((st = dbg_prologue("tact_dbg_bin_variance", p, n_units, workspace, workspace_bytes, &g,
                         &w)) != TACT_OK)
    return st;
  if (n_units == 0) return ok();
  if ((st = check_tensor(g, kv, g.n_entries, "kv")) != TACT_OK) return st;
  if ((st = check_buffer(var, "var", 4)) != TACT_OK) return st;
  launch_dct_tables(g, w.tab, stream);
  const StatsLayout sl = forward_stats(g, n_units, kv, g.n_entries, w, stream);
  // the allocation's own sum of the partials, scaled by 1/d, is the output
  launch_allocate2(g, n_units, w.var, var_stride(g), sl.parts, 1.0f / static_cast<float>(g.head_dim),
                   nullptr, RecordView{}, nullptr, nullptr, w.alloc, stream, sl.planes, var);
  return after_launch("tact_dbg_bin_variance");
}

tact_status tact_dbg_allocate(const tact_params* p, int64_t n_units, const float* var,
                              uint8_t* bits, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  Geometry g;
  Workspace w;
  tact_status st;
  if ((st = dbg_prologue("tact_dbg_allocate", p, n_units, workspace, workspace_bytes, &g, &w)) !=
      TACT_OK)
    return st;
  if (n_units == 0) return ok();
  if ((st = check_buffer(var, "var", 4)) != TACT_OK) return st;
  if ((st = check_buffer(bits, "bits", 1)) != TACT_OK) return st;
  RecordView none{};
  launch_allocate2(g, n_units, var, g.n_bins, 1, 1.0f, bits, none, nullptr, nullptr, w.alloc,
                   stream);
  return after_launch("tact_dbg_allocate");
}

tact_status tact_dbg_quantize(const tact_params* p, int64_t n_units, const float* coef,
                              const float* var, void* records, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  Geometry g;
  Workspace w;
  tact_status st;
  if ((st = dbg_prologue("tact_dbg_quantize", p, n_units, workspace, workspace_bytes, &g, &w)) !=
      TACT_OK)
    return st;
  if (g.rotation != TACT_ROTATION_NONE)
    return fail(TACT_ERR_UNSUPPORTED, "tact_dbg_quantize: the stage entry point codes the "
                "values as given; set rotation = TACT_ROTATION_NONE");
  if (g.quantizer != TACT_QUANT_LLOYD_MAX)
    return fail(TACT_ERR_UNSUPPORTED, "tact_dbg_quantize: the coding kernel uses the Lloyd-Max table");
  if (n_units == 0) return ok();
  if ((st = check_buffer(coef, "coef", 16)) != TACT_OK) return st;
  if ((st = check_buffer(var, "var", 4)) != TACT_OK) return st;
  if ((st = check_buffer(records, "records", 256)) != TACT_OK) return st;
  // the allocation writes the header, then the coding pass of the fused
  // path (which takes first planes and 1/gain from the header)
  const RecordView rv = view(g, records);
  launch_allocate2(g, n_units, var, g.n_bins, 1, 1.0f, nullptr, rv, nullptr, nullptr, w.alloc, stream);
  launch_quant(g, n_units, coef, g.n_entries, rv, stream);
  return after_launch("tact_dbg_quantize");
}

tact_status tact_dbg_dequantize(const tact_params* p, int64_t n_units, const void* records,
                                float* coef, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  Geometry g;
  Workspace w;
  tact_status st;
  if ((st = dbg_prologue("tact_dbg_dequantize", p, n_units, workspace, workspace_bytes, &g, &w)) !=
      TACT_OK)
    return st;
  if (g.rotation != TACT_ROTATION_NONE)
    return fail(TACT_ERR_UNSUPPORTED, "tact_dbg_dequantize: the stage entry point returns the "
                "coefficients without the inverse rotation; set rotation = TACT_ROTATION_NONE");
  if (n_units == 0) return ok();
  if ((st = check_buffer(records, "records", 256)) != TACT_OK) return st;
  if ((st = check_buffer(coef, "coef", 16)) != TACT_OK) return st;
  // the first decoding kernel of tact_decompress with identity matrices in
  // place of the DCT: its output is then g * level for every coefficient
  const RecordView rv = view(g, const_cast<void*>(records));
  launch_dct_tables(g, w.tab, stream, /*identity=*/7);
  launch_plane_offsets(g, n_units, rv, w.poff, stream);
  if (fused_path(g)) {
    launch_plane(g, n_units, 2, nullptr, coef, g.n_entries, w.tab, nullptr, 0, rv, w.poff, stream);
  } else {
    int ax[3];
    const int m = forward_axes(g, ax);
    launch_axis(g, n_units, ax[m - 1], 1, AX_PRO_DEQUANT, AX_EPI_F32, w.coef, g.n_entries, coef,
                g.n_entries, w.tab, nullptr, nullptr, 0, rv, w.poff, stream);
  }
  return after_launch("tact_dbg_dequantize");
}

}  // extern "C"
