// Device copy of the fixed Gaussian Lloyd-Max codebooks (1..8 bits, fp32,
// ascending), one private copy per translation unit that includes it.  The
// values are generated at build time by gen_codebooks.cpp.  Include inside
// namespace tact.
#ifndef TACT_CODEBOOK_DEVICE_H_
#define TACT_CODEBOOK_DEVICE_H_

#include "generated/codebooks.inc"

namespace {
// levels of the b-bit table start at (1 << b) - 2, thresholds at (1 << b) - b - 1
__constant__ float c_levels[TACT_CODEBOOK_LEVELS] = {TACT_CODEBOOK_LEVEL_VALUES};
__constant__ float c_thresholds[TACT_CODEBOOK_THRESHOLDS] = {TACT_CODEBOOK_THRESHOLD_VALUES};
// every quantizer, indexed by tact_params.quantizer: Lloyd-Max, uniform,
// NormalFloat (the last two for the absmax gain)
__constant__ float c_levels_q[3][TACT_CODEBOOK_LEVELS] = {
    {TACT_CODEBOOK_LEVEL_VALUES}, {TACT_UNIFORM_LEVEL_VALUES}, {TACT_NF_LEVEL_VALUES}};
__constant__ float c_thresholds_q[3][TACT_CODEBOOK_THRESHOLDS] = {
    {TACT_CODEBOOK_THRESHOLD_VALUES}, {TACT_UNIFORM_THRESHOLD_VALUES}, {TACT_NF_THRESHOLD_VALUES}};
}  // namespace

#endif  // TACT_CODEBOOK_DEVICE_H_
