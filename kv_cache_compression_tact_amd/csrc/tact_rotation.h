// The quantizer's shared rotation (page "TACT-KV: Tri-Axis Cosine Transform
// for Compressing Volumetric KV Caches in Medical VLMs", "Methodology in
// Plain English", stage 4): R = H_64 diag(s) / 8 on every 64-channel block of
// a bin, H_64 Sylvester's Hadamard matrix (H[j][j'] = (-1)^popcount(j & j')),
// s_j = -1 where the top bit of SplitMix64(seed + j) is set, else +1.
// Device helpers shared by the kernels; include inside namespace tact, after
// <stdint.h>.
#ifndef TACT_ROTATION_H_
#define TACT_ROTATION_H_

namespace {

constexpr uint64_t kRotationSeed = 0x54414354ull;

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014), one output per counter.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float rotation_sign(int j) {
  return (splitmix64(kRotationSeed + static_cast<uint64_t>(j)) >> 63) ? -1.0f : 1.0f;
}

}  // namespace

#endif  // TACT_ROTATION_H_
