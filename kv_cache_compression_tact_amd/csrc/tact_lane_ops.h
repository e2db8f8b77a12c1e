// Lane-level helpers shared by the matrix-core kernels (gfx950): column and
// row reductions over the MFMA fragment layout, and the 64-point
// Walsh-Hadamard butterflies of the quantizer's shared rotation (page
// "TACT-KV: Tri-Axis Cosine Transform for Compressing Volumetric KV Caches in
// Medical VLMs", "Methodology in Plain English", stage 4).  Include inside
// namespace tact's anonymous namespace.
#ifndef TACT_LANE_OPS_H_
#define TACT_LANE_OPS_H_

// max over the 4 lane groups that hold the K ranges of one column: the
// permlane swaps exchange lanes l and l ^ 32 (then l ^ 16) between two
// copies of v, so the max of the two results is the pairwise max
__device__ __forceinline__ float column_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the 16 lanes of each row (every lane gets the row sum): adds of
// rotated copies (DPP row rotate by 8, 4, 2, 1).
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xF, 0xF, true));
  return x;
}

// Partner values across the lanes of a 16-lane row: lane ^ 1, ^ 2 (quad
// permutes), ^ 4 (swizzle, bit mask mode), ^ 8 (row rotate by 8).
__device__ __forceinline__ float lane_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_xor4(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
}
__device__ __forceinline__ float lane_xor8(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
}

// Per-lane constants of the 16-point butterflies: sg[k] = -1 where lane bit
// k is set; the product of the four is the sign the butterflies leave.
struct LaneWht {
  float sg[4];
  float parity;    // (-1)^popcount(lane & 15)
  float parity8;   // (-1)^popcount(lane & 7)
  __device__ __forceinline__ explicit LaneWht(int lane) {
    parity = 1.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sg[k] = ((lane >> k) & 1) ? -1.f : 1.f;
      parity *= sg[k];
      if (k == 2) parity8 = parity;
    }
  }
};

// In-register butterflies over the 2 register bits, then the 4 lane
// butterflies.  A lane butterfly keeps x + sg * x_partner: where the lane
// bit is set that is x_self - x_partner, minus the Sylvester value, and the
// partner carries the same sign history, so the result is
// parity * (H_64 x) for each of the 4 values.
__device__ __forceinline__ void wht64(float& a0, float& a1, float& a2, float& a3,
                                      const LaneWht& w) {
  float b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
  a0 = b0 + b2;
  a2 = b0 - b2;
  a1 = b1 + b3;
  a3 = b1 - b3;
  float* v[4] = {&a0, &a1, &a2, &a3};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x = *v[q];
    x = fmaf(lane_xor1(x), w.sg[0], x);
    x = fmaf(lane_xor2(x), w.sg[1], x);
    x = fmaf(lane_xor4(x), w.sg[2], x);
    x = fmaf(lane_xor8(x), w.sg[3], x);
    *v[q] = x;
  }
}

#endif  // TACT_LANE_OPS_H_
