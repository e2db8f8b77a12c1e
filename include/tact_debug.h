/*
 * tact_debug.h -- stage entry points of the TACT-KV codec, for tests that
 * compare every step of the method (page "TACT-KV: Tri-Axis Cosine
 * Transform ...", section "Methodology in Plain English") with an
 * independent implementation.  Same conventions as tact.h: device pointers
 * owned by the caller, asynchronous on `stream`, validation before launch.
 * Per-unit arrays are packed one unit after another (no strides).
 */
#ifndef TACT_DEBUG_H_
#define TACT_DEBUG_H_

#include "tact.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stage 2.  inverse == 0: `in` holds n_units cache tensors of p->dtype,
 * `out` receives the fp32 DCT-II coefficients (same layout).  inverse != 0:
 * `in` holds fp32 coefficients, `out` the fp32 inverse transform (not
 * rounded).  Needs tact_dbg_workspace_bytes(p, n_units) of workspace. */
tact_status tact_dbg_dct3(const tact_params* p, int64_t n_units, int32_t inverse,
                          const void* in, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);
size_t tact_dbg_workspace_bytes(const tact_params* p, int64_t n_units);

/* Stage 3, first half: var[n_units * n_bins] from fp32 coefficients. */
tact_status tact_dbg_bin_variance(const tact_params* p, int64_t n_units,
                                  const float* coef, float* var,
                                  hipStream_t stream);

/* Stage 3, second half: bits[n_units * n_bins] (uint8) from variances. */
tact_status tact_dbg_allocate(const tact_params* p, int64_t n_units,
                              const float* var, uint8_t* bits,
                              hipStream_t stream);

/* Stage 4: quantize fp32 coefficients with the given gains and bits and
 * write complete records (gains, bits, group index, codes).  The bits of
 * each unit must sum to budget_bits * n_bins and not exceed max_bits; the
 * kernel does not check this (the caller's bits come from an allocation).
 * Quantizes the coefficients as they are: params->rotation must be
 * TACT_ROTATION_NONE (else TACT_ERR_UNSUPPORTED). */
tact_status tact_dbg_quantize(const tact_params* p, int64_t n_units,
                              const float* coef, const float* gains,
                              const uint8_t* bits, void* records,
                              hipStream_t stream);

/* Decoding, first step: the codes of every coefficient (uint8, same layout
 * as the unit tensor; 0 for zero-bit bins) read back from records. */
tact_status tact_dbg_unpack(const tact_params* p, int64_t n_units,
                            const void* records, uint8_t* codes,
                            hipStream_t stream);

/* Decoding, second step: dequantized fp32 coefficients g * level[code].
 * params->rotation must be TACT_ROTATION_NONE (else TACT_ERR_UNSUPPORTED). */
tact_status tact_dbg_dequantize(const tact_params* p, int64_t n_units,
                                const void* records, float* coef,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TACT_DEBUG_H_ */
