/*
 * tact_debug.h -- stage entry points of the TACT-KV codec, for tests that
 * compare every step of the method (page "TACT-KV: Tri-Axis Cosine
 * Transform for Compressing Volumetric KV Caches in Medical VLMs", section
 * "Methodology in Plain English") with an independent implementation.
 *
 * Every call runs the kernels that tact_compress and tact_decompress launch
 * for the same geometry, stopped after (or started at) the named step, so
 * the step is checked as the codec computes it.  Same conventions as tact.h:
 * device pointers owned by the caller, asynchronous on `stream`, validation
 * before any launch, TACT_ERR_* on failure with detail in tact_last_error().
 * Per-unit arrays are packed one unit after another (no strides); one call
 * covers at most 65535 units.  Calls that take a workspace need
 * tact_dbg_workspace_bytes(p, n_units) bytes of it, 256-byte aligned.
 */
#ifndef TACT_DEBUG_H_
#define TACT_DEBUG_H_

#include "tact.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace of the stage calls for n_units units (0 for invalid params or a
 * unit count outside 1..65535). */
size_t tact_dbg_workspace_bytes(const tact_params* p, int64_t n_units);

/* Stage 2, the separable orthonormal DCT-II along the axes in p->axes,
 * without the quantizer's rotation (p->rotation is ignored).
 * inverse == 0: `in` holds n_units cache tensors of p->dtype, `out` receives
 * the fp32 coefficients (same layout), computed by the coding path's passes:
 * for the fused layout (all three axes, H and W up to 32, the Lloyd-Max
 * quantizer) the S pass and the H/W plane pass; otherwise the axis passes.
 * inverse != 0: `in` holds fp32 coefficients, `out` the fp32 inverse
 * transform (not rounded), by the axis passes of the decoding path. */
tact_status tact_dbg_dct3(const tact_params* p, int64_t n_units, int32_t inverse,
                          const void* in, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Stage 3, first half: var[n_units * n_bins] (fp32, bin order), the per-bin
 * second moments over head_dim of the coefficients of the cache tensors `kv`
 * (p->dtype, packed), exactly as the allocation of tact_compress reads them:
 * the forward passes with their sums-of-squares epilogue (and the
 * quantizer's rotation when p->rotation asks for it), then the allocation
 * kernel's sum of the partials. */
tact_status tact_dbg_bin_variance(const tact_params* p, int64_t n_units, const void* kv,
                                  float* var, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Stage 3, second half: bits[n_units * n_bins] (uint8) from variances
 * var[n_units * n_bins] (fp32), by the allocation kernels of tact_compress
 * (the workspace holds their scratch). */
tact_status tact_dbg_allocate(const tact_params* p, int64_t n_units,
                              const float* var, uint8_t* bits, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Stage 4: complete records (gains, bits, group index, codes) of the fp32
 * coefficients `coef` (n_units unit tensors, packed) with the allocation of
 * the variances var[n_units * n_bins]: the allocation kernel writes the
 * header (gain = sqrt(var), fp32), the coding kernel of the fused layout the
 * codes.  The values are coded as given: params->rotation must be
 * TACT_ROTATION_NONE and params->quantizer TACT_QUANT_LLOYD_MAX (else
 * TACT_ERR_UNSUPPORTED). */
tact_status tact_dbg_quantize(const tact_params* p, int64_t n_units,
                              const float* coef, const float* var,
                              void* records, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Decoding, first step: the dequantized coefficients g * level[code] (fp32,
 * same layout as the unit tensor; 0 for zero-bit bins) of n_units records,
 * by the first decoding kernel of tact_decompress (the H/W plane pass of the
 * fused layout, else the last forward axis) with identity matrices in place
 * of the DCT.  The values carry that kernel's split-fp16 rounding (relative
 * error below 2^-19), far below the spacing of the levels, so the codes
 * follow from them exactly.  params->rotation must be TACT_ROTATION_NONE
 * (else TACT_ERR_UNSUPPORTED). */
tact_status tact_dbg_dequantize(const tact_params* p, int64_t n_units,
                                const void* records, float* coef,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TACT_DEBUG_H_ */
