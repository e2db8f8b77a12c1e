/*
 * tact.h -- C ABI of the TACT-KV visual-KV-cache codec for AMD Instinct
 * MI355X (gfx950).
 *
 * The codec follows the AI-summary page "TACT-KV: Tri-Axis Cosine Transform
 * for Compressing Volumetric KV Caches in Medical VLMs", section
 * "Methodology in Plain English" (stages 1-4 and the decoding paragraph).
 * Per unit -- one layer, one sequence, the K or the V tensor -- it:
 *   1. views the visual span of the cache as an (S, H, W, kv_heads, head_dim)
 *      volume on the vision encoder's grid                       (stage 1);
 *   2. applies a separable orthonormal DCT-II along S, H and W   (stage 2);
 *   3. estimates each frequency bin's variance from the unit itself and
 *      splits the unit's bit budget over the bins by reverse water-filling,
 *      capped at max_bits per bin, hitting the budget exactly   (stage 3);
 *   4. quantizes each bin with a gain (its RMS, stored as fp32) and a fixed
 *      Gaussian Lloyd-Max codebook at the bin's bit width        (stage 4);
 * and decoding reverses the steps (dequantize, inverse DCT, round).
 *
 * Definitions used throughout:
 *   bin      one (ks, kh, kw, head) frequency of one head; flat bin index
 *            ((ks*H + kh)*W + kw)*kv_heads + head.  n_bins = S*H*W*kv_heads.
 *   variance (1/head_dim) * sum_j c_j^2 over the bin's head_dim coefficients.
 *   budget   T = budget_bits * n_bins bit-planes per unit; bin i gets b_i
 *            planes with sum_i b_i = T and 0 <= b_i <= max_bits.  The b_i are
 *            the T largest marginal gains var_i * 4^-(k-1) (1 <= k <= max_bits)
 *            ordered by (gain desc, bin asc, k asc) -- the result of
 *            bisection for the water level plus the +-1 greedy correction.
 *   code     u = fl32(c * fl32(1/g)) with g = fl32(sqrt(variance)) (u = 0 when
 *            g == 0); code = number of fp32 Lloyd-Max thresholds <= u.
 *
 * Memory.  All buffer arguments are DEVICE pointers owned by the caller; the
 * library never allocates, frees or synchronizes.  Work is enqueued on the
 * given HIP stream and runs asynchronously; the return value reports only
 * argument validation and launch errors.  Arguments are validated before any
 * HIP call: an invalid call launches nothing.  Buffers must not overlap
 * unless stated.  Inputs must be finite.
 *
 * Unit tensor layout: row-major (S, H, W, kv_heads, head_dim), element type
 * given by tact_params.dtype; consecutive units are unit_stride elements
 * apart (unit_stride >= S*H*W*kv_heads*head_dim, a multiple of 8).  Tensor
 * pointers must be 16-byte aligned; records and workspace 256-byte aligned.
 *
 * Record layout (one per unit, tact_record_bytes() bytes, regions 256-byte
 * aligned, in this order):
 *   gains  float32[n_bins]               per-bin gain g
 *   bits   uint8[n_bins]                 b_i
 *   groups uint32[ceil(n_bins/64)]       sum_{k < 64*g} b_k (first plane of
 *                                        every 64th bin)
 *   codes  uint64[T*head_dim/64]         bin i's plane q (q = 0 is the least
 *                                        significant code bit) starts at bit
 *                                        (sum_{k<i} b_k + q) * head_dim; bit j
 *                                        of a plane is bit q of code_j.
 * The record is position independent: it can be copied or stored as is.
 * Decoding (tact_decompress, tact_attend) locates each bin's planes from the
 * group index and the bit widths, so the index must agree with the widths,
 * as it does in every record tact_compress writes.  A record whose index or
 * widths are inconsistent decodes to unspecified values, but never makes a
 * kernel read or write outside the record, the output or the workspace:
 * widths above max_bits, and planes that would run past the T planes of the
 * record, decode as zero.
 */
#ifndef TACT_H_
#define TACT_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TACT_OK = 0,
  TACT_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad alignment  */
  TACT_ERR_UNSUPPORTED = 2,      /* valid C call, geometry not supported   */
  TACT_ERR_WORKSPACE = 3,        /* workspace missing or too small         */
  TACT_ERR_HIP = 4               /* the HIP runtime reported an error      */
} tact_status;

typedef enum { TACT_BF16 = 0, TACT_F32 = 1 } tact_dtype;

/* Transform axes (bit mask); the method transforms all three.  Subsets are
 * the transform ablation of the page's "Main Findings"; 0 (TACT_AXES_NONE)
 * codes the tokens without a transform (each bin is one token of one head). */
enum { TACT_AXES_NONE = 0, TACT_AXIS_S = 1, TACT_AXIS_H = 2, TACT_AXIS_W = 4, TACT_AXES_ALL = 7 };

/* Allocation mode: 0 = reverse water-filling (the method); 1 = uniform, every
 * bin budget_bits planes (the page's "uniform allocation" ablation). */
enum { TACT_ALLOC_WATERFILL = 0, TACT_ALLOC_UNIFORM = 1 };

/* The quantizer's fixed shared rotation (section "Methodology in Plain
 * English", stage 4: the gain-normalized bin vector is rotated by one fixed
 * orthogonal matrix before scalar quantization, and rotated back after
 * dequantization).  TACT_ROTATION_HADAMARD (the method) is
 * R = H_64 diag(s) / 8 on every 64-channel block of a bin: H_64 is
 * Sylvester's Hadamard matrix, H[j][j'] = (-1)^popcount(j & j'), and s_j is
 * -1 where the top bit of SplitMix64(0x54414354 + j) is set, else +1
 * (SplitMix64: Steele, Lea and Flood, 2014).  Code bit j of a word is the
 * cell of the rotated coordinate j.  TACT_ROTATION_NONE quantizes the
 * normalized coefficients themselves (an ablation). */
enum { TACT_ROTATION_NONE = 0, TACT_ROTATION_HADAMARD = 1 };

/* Scalar quantizer of the coded bins ("Main Findings", the comparison of
 * quantizer backends).  TACT_QUANT_LLOYD_MAX (the method): gain = RMS of the
 * bin, Gaussian Lloyd-Max table.  TACT_QUANT_UNIFORM: gain = largest |value|
 * of the (rotated) bin vector, 2^b equal cells of [-1, 1] with levels at the
 * cell centres.  TACT_QUANT_NF: the same gain, NormalFloat levels (normal
 * quantiles at (k + 1/2) / 2^b, outermost levels +-1).  Thresholds are the
 * midpoints of adjacent levels; the allocation is the same for all three.
 * The two comparison backends run on the per-axis kernels. */
enum { TACT_QUANT_LLOYD_MAX = 0, TACT_QUANT_UNIFORM = 1, TACT_QUANT_NF = 2 };

typedef struct {
  /* A unit is S * H * W * kv_heads * head_dim entries.  With each of S, H
   * and W rounded up to 16, 32 or 64 (the first that holds it), the padded
   * unit in fp32, 4 * S' * H' * W' * kv_heads * head_dim bytes, must not
   * exceed 2^30 bytes (so at most 2^28 entries per unit); larger units are
   * TACT_ERR_UNSUPPORTED. */
  int32_t S, H, W;      /* grid of the vision encoder, each 1..64            */
  int32_t kv_heads;     /* 1..64                                             */
  int32_t head_dim;     /* 64, 128 or 256                                    */
  int32_t budget_bits;  /* average code bits per entry, 0..max_bits          */
  int32_t max_bits;     /* per-bin cap, 1..8 (the page caps at 8)            */
  int32_t dtype;        /* tact_dtype of the cache tensors (in == out)       */
  int32_t axes;         /* TACT_AXES_ALL, a subset, or TACT_AXES_NONE        */
  int32_t alloc_mode;   /* TACT_ALLOC_WATERFILL or TACT_ALLOC_UNIFORM        */
  int32_t rotation;     /* TACT_ROTATION_HADAMARD or TACT_ROTATION_NONE      */
  int32_t quantizer;    /* TACT_QUANT_LLOYD_MAX, _UNIFORM or _NF             */
} tact_params;

/* Fills *p with the method's defaults for the given geometry and budget
 * (dtype bf16, all axes, water-filling, cap 8, Hadamard rotation,
 * Lloyd-Max quantizer). */
void tact_params_init(tact_params* p, int32_t S, int32_t H, int32_t W,
                      int32_t kv_heads, int32_t head_dim, int32_t budget_bits);

/* Bytes of one unit's record; 0 if *p is invalid (see tact_last_error). */
size_t tact_record_bytes(const tact_params* p);

/* Workspace bytes that tact_compress / tact_decompress / tact_roundtrip need
 * for a call over n_units units (a larger workspace is accepted); 0 if *p is
 * invalid.  The stage entry points of tact_debug.h need none unless stated. */
size_t tact_workspace_bytes(const tact_params* p, int64_t n_units);

/* Compress n_units units: kv (device, unit_stride elements apart) ->
 * records (device, n_units * tact_record_bytes(p) bytes, one after another).
 * Stages 1-4 of the method.  n_units == 0 is a no-op. */
tact_status tact_compress(const tact_params* p, int64_t n_units,
                          const void* kv, int64_t kv_unit_stride,
                          void* records, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Decompress n_units records into kv_out (same layout rules as kv):
 * unpack, dequantize, inverse DCT, round to bf16 (nearest even) or fp32. */
tact_status tact_decompress(const tact_params* p, int64_t n_units,
                            const void* records, void* kv_out,
                            int64_t out_unit_stride, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* tact_compress followed by tact_decompress.  records may be NULL, in which
 * case the records are kept in the workspace (tact_workspace_bytes then
 * includes them).  kv_out may equal kv (in place). */
tact_status tact_roundtrip(const tact_params* p, int64_t n_units,
                           const void* kv, int64_t kv_unit_stride,
                           void* kv_out, int64_t out_unit_stride,
                           void* records, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* tact_roundtrip for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  It
 * takes no workspace argument: the workspace is a library-owned static
 * device array of TACT_STATIC_WORKSPACE_BYTES, one per GPU, held from the
 * library's first use on that GPU until the process ends, and the call
 * allocates nothing.  Same arguments, results (bit for bit), aliasing rules
 * and errors as tact_roundtrip; a batch runs as many units per chunk as the
 * array holds.  Geometries whose single unit needs more workspace than the
 * array (tact_workspace_bytes(p, 1) > TACT_STATIC_WORKSPACE_BYTES; the
 * 64 x 24 x 24 x 8 x 128 unit needs about 163 MB) are rejected with
 * TACT_ERR_UNSUPPORTED before anything is enqueued.  Every call on one GPU
 * uses that GPU's one array: calls that overlap on a GPU (other streams,
 * other host threads) race and must be serialized by the caller.  No part of
 * the array needs to start at zero: each kernel writes what a later one
 * reads. */
#define TACT_STATIC_WORKSPACE_BYTES ((size_t)192 << 20)
tact_status tact_roundtrip_noalloc(const tact_params* p, int64_t n_units,
                                   const void* kv, int64_t kv_unit_stride,
                                   void* kv_out, int64_t out_unit_stride,
                                   void* records, hipStream_t stream);

/* ---- Decoding fused into attention --------------------------------------
 * The page's decoding paragraph ("Methodology in Plain English") allows the
 * decoder to live inside the attention kernel: tact_attend reads only the
 * records and writes no decoded cache.  It runs one decoding step of
 * attention over the visual tokens of n_pairs unit pairs -- the K record and
 * the V record of one layer and sequence, both coded with *p -- reading only
 * the records:
 *   k_records, v_records  device, n_pairs records each, tact_record_bytes(p)
 *            apart (as tact_compress writes them), 256-byte aligned;
 *   q        device float32 [n_pairs][q_heads][head_dim]; query head r reads
 *            kv head r / (q_heads / kv_heads) (grouped heads);
 *   out      device float32 [n_pairs][q_heads][head_dim]:
 *            out = sum_t p_t v_t over the S*H*W visual tokens t, with
 *            p_t = exp(scale * q . k_t - lse) (the softmax over those tokens);
 *   lse      device float32 [n_pairs][q_heads]: log sum_t exp(scale * q . k_t),
 *            which merges the result with attention over the text tokens;
 * where k_t, v_t are the decoded cache: the values tact_decompress
 * reconstructs, before the output rounding.  The inverse DCT is linear, so
 * the scores are the inverse 3-D DCT of the per-bin projections q . c_f and
 * the output is the sum over coded V bins of DCT3(p)_f c_f; only coded bins
 * are read.  Limits (TACT_ERR_UNSUPPORTED otherwise): q_heads a multiple of
 * kv_heads with at most 16 query heads per kv head, S*H*W <= 40000.  q, out
 * and lse are 4-byte aligned and must not overlap; n_pairs == 0 is a no-op.
 * Precision: fp32 throughout (see the tests for the bound). */
size_t tact_attend_workspace_bytes(const tact_params* p, int64_t n_pairs, int32_t q_heads);
tact_status tact_attend(const tact_params* p, int64_t n_pairs, int32_t q_heads,
                        const void* k_records, const void* v_records, const float* q,
                        float scale, float* out, float* lse, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* tact_status_string(tact_status s);

/* Detail of the last failed call on this thread ("" if none). */
const char* tact_last_error(void);

/* Host-side copy of the library's fp32 Lloyd-Max table at `bits` (1..8):
 * 2^bits levels and 2^bits - 1 thresholds, ascending.  Either pointer may be
 * NULL.  Returns the number of levels, or 0 for an invalid bit width. */
int32_t tact_codebook(int32_t bits, float* levels, float* thresholds);

/* The same for any quantizer (tact_params.quantizer); 0 for an invalid
 * quantizer or bit width. */
int32_t tact_quantizer_table(int32_t quantizer, int32_t bits, float* levels, float* thresholds);

#ifdef __cplusplus
}
#endif

#endif /* TACT_H_ */
