// Internal interface between the C-ABI host layer (tact_api.cpp) and the
// gfx950 kernels (tact_mfma.hip, tact_quant.hip, tact_attend.hip).  Not
// installed, not part of the ABI.
#ifndef TACT_INTERNAL_H_
#define TACT_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "tact.h"

namespace tact {

// Geometry of one unit and of its record, derived from validated params.
struct Geometry {
  int S, H, W, kv_heads, head_dim;
  int max_bits, budget_bits, axes, alloc_mode, rotation, quantizer;
  int dtype;
  int64_t n_bins;        // S*H*W*kv_heads
  int64_t n_entries;     // n_bins * head_dim
  int64_t total_bits;    // T = budget_bits * n_bins (bit-planes)
  int64_t n_groups;      // ceil(n_bins / 64)
  // record layout (bytes from the record start)
  int64_t off_gains, off_bits, off_groups, off_codes, code_bytes, record_bytes;
};

// Locations of the record regions for a batch of units.
struct RecordView {
  uint8_t* base;         // record of unit 0
  int64_t stride;        // bytes between records
  int64_t off_gains, off_bits, off_groups, off_codes;
};

constexpr int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

// ---- launchers; all asynchronous on `stream` --------------------------------
// Prologue / epilogue selectors of launch_axis.
enum { AX_PRO_BF16 = 0, AX_PRO_F32 = 1, AX_PRO_DEQUANT = 2 };
enum { AX_EPI_F32 = 0, AX_EPI_BF16 = 1, AX_EPI_STATS = 2, AX_EPI_QUANT = 3 };
constexpr int64_t kDctTableFloats = 3 * 64 * 64;

// DCT-II matrices of the three axes into tab[3][64][64] (fp32, zero padded).
// Bit a of `identity` puts the identity in place of axis a's matrix; the
// default (-1) does so for the S axis of a geometry that transforms no axis.
void launch_dct_tables(const Geometry& g, float* tab, hipStream_t stream, int identity = -1);

// One axis (0 = S, 1 = H, 2 = W) of the transform on the matrix cores over
// n_units units; see tact_mfma.hip for the prologue / epilogue contracts.
// When the geometry rotates: rot_in makes a plain fp32 pass apply the
// inverse of the quantizer's rotation to its input rows, rot_out makes a
// plain pass with fp32 output apply the rotation to its output rows (the
// rotation acts on the channels and commutes with the transform).
void launch_axis(const Geometry& g, int64_t n_units, int axis, int inverse, int pro, int epi,
                 const void* in, int64_t in_stride, void* out, int64_t out_stride,
                 const float* tab, float* var, const float* inv_gain, int64_t var_stride,
                 RecordView rec, const uint32_t* plane_off, hipStream_t stream,
                 bool rot_in = false, bool rot_out = false);

// Allocation by exact radix selection; writes bits_out and/or the record
// header, per-bin first planes into plane_off, reciprocal gains into
// inv_gain (stride var_stride) and the variances it allocated from into
// var_out ([u][bin]); each may be null.  var holds `parts` partial sums per
// bin, scaled by var_scale: consecutive per bin, or (planes) stored plane by
// plane as the plane pass writes them, [slab][s][kh][kw] per unit.  Each unit
// runs on up to kAllocMaxSlices workgroups; scratch (kAllocScratchBytes per
// unit, 256-byte aligned) holds their shared histograms and totals.
constexpr int kAllocMaxSlices = 64;
constexpr int64_t kAllocScratchBytes = 4 * 8192 + 256 + 16 * kAllocMaxSlices;
void launch_allocate2(const Geometry& g, int64_t n_units, const float* var, int64_t var_stride,
                      int parts, float var_scale, uint8_t* bits_out, RecordView rec,
                      uint32_t* plane_off, float* inv_gain, void* scratch, hipStream_t stream,
                      bool planes = false, float* var_out = nullptr);

// Fused H and W axes (see tact_mfma.hip); mode 0 = forward: coefficients
// to `out` (may equal `in`) and variance partial sums; 2 = decode + inverse.
bool plane_supported(const Geometry& g);
void launch_plane(const Geometry& g, int64_t n_units, int mode, const float* in, float* out,
                  int64_t ustride, const float* tab, float* var_part, int64_t var_stride,
                  RecordView rec, const uint32_t* plane_off, hipStream_t stream);

// Quantize + pack the final coefficients coef ([u][bin][head_dim], unit
// stride ustride; already rotated when the geometry rotates) into the
// records, whose header (gains, bits, group index) the allocation has
// written (tact_quant.hip).
void launch_quant(const Geometry& g, int64_t n_units, const float* coef, int64_t ustride,
                  RecordView rec, hipStream_t stream);

// Per-bin first planes of n_units records (from each record's group index
// and bit widths); with rec2, also those of n_units records of rec2 into
// plane_off2, in the same launch.
void launch_plane_offsets(const Geometry& g, int64_t n_units, RecordView rec,
                          uint32_t* plane_off, hipStream_t stream,
                          const RecordView* rec2 = nullptr, uint32_t* plane_off2 = nullptr);

// Decoding fused into attention (tact_attend.hip): per unit pair the
// projections, the field transforms and softmax, the output partial sums per
// chunk of bins, and the final sum and inverse rotation.  Workspace: tab
// (DCT tables, filled by launch_dct_tables), frags (the tables as split fp16
// MFMA fragments, kAttendFragBytes), the per-bin first planes of both record
// arrays, qrot [pairs][q_heads][d],
// field [pairs][q_heads][S*H*W], partial [pairs][kv_heads][chunks][rep][d].
int attend_chunks(const Geometry& g);
// 3 axes x 2 directions x 4 row tiles x 2 K steps x (hi, lo) x 64 lanes x 16 B
// query heads per kv head that tact_attend accepts (its kernels are
// specialised for capacities up to this)
constexpr int kMaxAttendRep = 16;
constexpr int64_t kAttendFragBytes = 3 * 2 * 4 * 2 * 2 * 64 * 16;
void launch_attend(const Geometry& g, int64_t n_pairs, int q_heads, RecordView krec,
                   RecordView vrec, const uint32_t* kpoff, const uint32_t* vpoff, const float* q,
                   float scale, float* qrot, float* field, float* partial, float* out, float* lse,
                   const float* tab, uint32_t* frags, hipStream_t stream);

// Device address of the current GPU's copy of the library-owned workspace
// (TACT_STATIC_WORKSPACE_BYTES, 256-byte aligned; tact_static_ws.hip),
// looked up on the first call on each GPU.
hipError_t static_workspace(void** ptr);

// Host copy of the fp32 codebooks (Lloyd-Max), and of every quantizer's,
// indexed [quantizer][...] (tact_codebooks.cpp).
extern const float kHostLevels[];
extern const float kHostThresholds[];
extern const float* const kHostLevelsQ[3];
extern const float* const kHostThresholdsQ[3];

}  // namespace tact

#endif  // TACT_INTERNAL_H_
