// Host copies of the fixed scalar codebooks (page "TACT-KV: Tri-Axis Cosine
// Transform for Compressing Volumetric KV Caches in Medical VLMs", section
// "Methodology in Plain English", stage 4): the Gaussian Lloyd-Max tables
// and the two absmax backends of the quantizer comparison, fp32, ascending,
// 1..8 bits.  The values are generated at build time by gen_codebooks.cpp;
// tact_quantizer_table hands them to callers.
#include "tact_internal.h"

namespace tact {

#include "generated/codebooks.inc"

const float kHostLevels[TACT_CODEBOOK_LEVELS] = {TACT_CODEBOOK_LEVEL_VALUES};
const float kHostThresholds[TACT_CODEBOOK_THRESHOLDS] = {TACT_CODEBOOK_THRESHOLD_VALUES};
static const float kHostUniformLevels[TACT_CODEBOOK_LEVELS] = {TACT_UNIFORM_LEVEL_VALUES};
static const float kHostUniformThresholds[TACT_CODEBOOK_THRESHOLDS] = {TACT_UNIFORM_THRESHOLD_VALUES};
static const float kHostNfLevels[TACT_CODEBOOK_LEVELS] = {TACT_NF_LEVEL_VALUES};
static const float kHostNfThresholds[TACT_CODEBOOK_THRESHOLDS] = {TACT_NF_THRESHOLD_VALUES};
const float* const kHostLevelsQ[3] = {kHostLevels, kHostUniformLevels, kHostNfLevels};
const float* const kHostThresholdsQ[3] = {kHostThresholds, kHostUniformThresholds, kHostNfThresholds};

}  // namespace tact
