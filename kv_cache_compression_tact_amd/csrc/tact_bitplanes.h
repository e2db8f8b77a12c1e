// Bit planes to codes: the record stores a bin's codes as bit planes (bit c
// of plane k is bit k of channel c's code, page "TACT-KV: Tri-Axis Cosine
// Transform for Compressing Volumetric KV Caches in Medical VLMs",
// "Methodology in Plain English", stage 4, in this library's record
// layout).  Decoders that need one code per channel turn NB planes of 32
// channels into 32 byte-sized codes: a 4x4 byte transpose of the planes on
// v_perm_b32 (the planes' byte j gathered into one 64-bit row block per 8
// channels), then an 8x8 bit transpose of each block by three delta swaps
// (H. S. Warren, Hacker's Delight, 2nd ed., section 7-3).  Planes at or past
// NB must not be passed; a bin narrower than NB has zero planes there.
// Include inside namespace tact's anonymous namespace, after <stdint.h>.
#ifndef TACT_BITPLANES_H_
#define TACT_BITPLANES_H_

// 8x8 bit matrix in a 64-bit word, row r = byte r, column c = bit c of the
// byte: returns its transpose (bit 8r + c <-> bit 8c + r)
__device__ __forceinline__ uint64_t transpose8x8(uint64_t x) {
  uint64_t t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
  x = x ^ t ^ (t << 7);
  t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
  x = x ^ t ^ (t << 14);
  t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
  return x ^ t ^ (t << 28);
}

// byte j of p0..p3 into o[j] = (p0.b_j, p1.b_j, p2.b_j, p3.b_j)
__device__ __forceinline__ void byte_transpose4(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                                uint32_t (&o)[4]) {
  // v_perm_b32 picks bytes 0..3 from its second operand and 4..7 from its
  // first: a0 = (p0.b0, p1.b0, p0.b1, p1.b1), a1 = (p0.b2, p1.b2, p0.b3, p1.b3)
  const uint32_t a0 = __builtin_amdgcn_perm(p1, p0, 0x05010400u);
  const uint32_t a1 = __builtin_amdgcn_perm(p1, p0, 0x07030602u);
  const uint32_t b0 = __builtin_amdgcn_perm(p3, p2, 0x05010400u);
  const uint32_t b1 = __builtin_amdgcn_perm(p3, p2, 0x07030602u);
  o[0] = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
}

// q[t] byte i = the code of channel 4 t + i, from planes p[0..NB-1] of 32
// channels (NB = 1, 2, 4 or 8)
template <int NB>
__device__ __forceinline__ void planes_to_codes(const uint32_t* p, uint32_t (&q)[8]) {
  static_assert(NB == 1 || NB == 2 || NB == 4 || NB == 8, "plane count");
  uint32_t lo[4], hi[4] = {0u, 0u, 0u, 0u};
  if constexpr (NB == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) lo[j] = __builtin_amdgcn_perm(0u, p[0], 0x0c0c0c00u + j);
  } else if constexpr (NB == 2) {
    // (p0.b_j, p1.b_j, 0, 0); selector 0x0c gives a zero byte
#pragma unroll
    for (int j = 0; j < 4; ++j) lo[j] = __builtin_amdgcn_perm(p[1], p[0], 0x0c0c0400u + 0x0101u * j);
  } else {
    byte_transpose4(p[0], p[1], p[2], p[3], lo);
    if constexpr (NB == 8) byte_transpose4(p[4], p[5], p[6], p[7], hi);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t x = transpose8x8((static_cast<uint64_t>(hi[j]) << 32) | lo[j]);
    q[2 * j] = static_cast<uint32_t>(x);
    q[2 * j + 1] = static_cast<uint32_t>(x >> 32);
  }
}

#endif  // TACT_BITPLANES_H_
