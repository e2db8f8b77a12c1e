// Coding pass of the TACT-KV codec for gfx950 (page "TACT-KV: Tri-Axis
// Cosine Transform for Compressing Volumetric KV Caches in Medical VLMs",
// section "Methodology in Plain English", stage 4): gain-shape scalar
// quantization of the final DCT coefficients and bit-plane packing.
//
// k_quant streams the coefficient volume once, reading only bins that were
// given bits.  One wave owns 64 consecutive bins of a unit (lane j holds
// bin j's bit width, first plane and 1/gain) and walks them one at a time:
// lane c is channel c of a 64-channel word, so a bin's codes for one bit
// plane are one ballot.  The cell index is found most significant bit
// first (binary search over the sorted thresholds), and the ballot of each
// step is directly the word of that bit plane.  Words are gathered into
// lanes (word k in lane k) with their record offsets and written up to 64
// at a time.
#include <hip/hip_runtime.h>

#include "tact_internal.h"

namespace tact {

#include "codebook_device.h"

namespace {

constexpr int kWave = 64;
constexpr int kQuantWaves = 4;

// ---- the shared rotation, lane = channel ------------------------------------
// R = H_64 diag(s) / 8 with Sylvester's H_64 (H[j][j'] = (-1)^popcount(j&j'))
// and s_j = -1 where the top bit of SplitMix64(0x54414354 + j) is set.
constexpr uint64_t kRotationSeed = 0x54414354ull;

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Butterfly on lane bit k: y = x + sg_k * x[lane ^ 2^k], where sg_k = -1
// on lanes whose bit k is set.  On those lanes that is the negated
// Sylvester value, and both lanes of a pair carry the same sign history,
// so after the six stages y = (-1)^popcount(lane) (H_64 x)[lane].
__device__ __forceinline__ float wht64_lanes(float x, const float (&sg)[6]) {
  const int xi = __float_as_int(x);
  x = fmaf(__int_as_float(__builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, true)), sg[0], x);
  x = fmaf(__int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)), sg[1], x);
  x = fmaf(__int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F)), sg[2], x);
  x = fmaf(__int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true)), sg[3], x);
  // lanes l and l ^ 16 (l ^ 32) by a permlane swap of two copies: the first
  // result holds the even (lower) partner, the second the odd (upper) one
  {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaf(__uint_as_float(r[0]), sg[4], __uint_as_float(r[1]));
  }
  {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaf(__uint_as_float(r[0]), sg[5], __uint_as_float(r[1]));
  }
  return x;
}

struct QuantArgs {
  const float* coef;         // final DCT coefficients, [u][bin][head_dim]
  int64_t ustride;           // elements between units
  int64_t n_bins, total_bits;
  int head_dim, max_bits;
  const float* inv_gain;     // fp32 1/gain per bin (0 for gain 0)
  int64_t var_stride;        // floats per unit in inv_gain
  const uint32_t* plane_off; // first bit plane of each bin, [u][bin]
  RecordView rec;
  int rotate;
};

__global__ __launch_bounds__(kWave * kQuantWaves) void k_quant(QuantArgs a) {
  __shared__ float s_thr[TACT_CODEBOOK_THRESHOLDS];
  for (int j = threadIdx.x; j < TACT_CODEBOOK_THRESHOLDS; j += blockDim.x) s_thr[j] = c_thresholds[j];
  __syncthreads();
  const int lane = threadIdx.x % kWave;
  const int64_t u = blockIdx.y;
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * kQuantWaves + threadIdx.x / kWave) * kWave;
  if (b0 >= a.n_bins) return;
  const int wpp = a.head_dim / 64;

  // side info of bin b0 + lane
  int bj = 0, pj = 0;
  float ij = 0.f;
  if (b0 + lane < a.n_bins) {
    const int64_t bin = b0 + lane;
    const uint8_t* bits = a.rec.base + u * a.rec.stride + a.rec.off_bits;
    bj = bits[bin];
    pj = static_cast<int>(a.plane_off[u * a.n_bins + bin]);
    ij = a.inv_gain[u * a.var_stride + bin];
    if (bj > a.max_bits || static_cast<int64_t>(static_cast<uint32_t>(pj)) + bj > a.total_bits) bj = 0;
  }

  // rotation constants of lane (channel) c: the butterfly signs, s_c, and
  // the output factor (-1)^popcount(c) / 8
  float sg[6];
  float s_in = 1.f, r_out = 1.f;
  if (a.rotate) {
    float par = 1.f;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      sg[k] = ((lane >> k) & 1) ? -1.f : 1.f;
      par *= sg[k];
    }
    s_in = (splitmix64(kRotationSeed + static_cast<uint64_t>(lane)) >> 63) ? -1.f : 1.f;
    r_out = 0.125f * par;
  }

  const float* cu = a.coef + u * a.ustride + b0 * a.head_dim + lane;
  uint64_t* words = reinterpret_cast<uint64_t*>(a.rec.base + u * a.rec.stride + a.rec.off_codes);
  // gathered words: lane k holds word k and its index in the record
  uint32_t wlo = 0, whi = 0, widx = 0;
  int cnt = 0;
  auto flush = [&]() {
    if (lane < cnt) words[widx] = (static_cast<uint64_t>(whi) << 32) | wlo;
    cnt = 0;
  };

  // coded bins of this wave, lowest first; the words of the next one are
  // fetched while the current one is quantized (up to 4 per bin)
  uint64_t todo = __ballot(bj > 0);
  float nxt[4] = {0.f, 0.f, 0.f, 0.f};
  auto fetch = [&](int j) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (h < wpp) nxt[h] = cu[j * a.head_dim + 64 * h];
  };
  if (todo) fetch(__builtin_ctzll(todo));
  while (todo) {
    const int j = __builtin_ctzll(todo);
    todo &= todo - 1;
    float cur[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) cur[h] = nxt[h];
    if (todo) fetch(__builtin_ctzll(todo));
    const int b = __builtin_amdgcn_readlane(bj, j);
    const uint32_t p0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(pj, j));
    const float inv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ij), j));
    const float* t = s_thr + ((1 << b) - b - 1);            // 2^b - 1 sorted thresholds
    // the table is symmetric: its middle threshold is 0 and the two next
    // split points are -t2 and +t2
    const float t2 = b > 1 ? t[(3 << (b - 2)) - 1] : 0.f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (h >= wpp) break;
      float v = cur[h];
      if (a.rotate) v = wht64_lanes(v * s_in, sg) * (inv * r_out);
      else v = v * inv;
      if (cnt + b > kWave) flush();
      // most significant bit first: step k compares with the threshold that
      // splits the remaining cells; the ballot is bit plane k's word
      auto stage = [&](uint64_t wd, int k) {
        if (lane == cnt) {
          wlo = static_cast<uint32_t>(wd);
          whi = static_cast<uint32_t>(wd >> 32);
          widx = (p0 + static_cast<uint32_t>(k)) * wpp + h;
        }
        ++cnt;
      };
      bool up = 0.f <= v;
      stage(__ballot(up), b - 1);
      int idx = up ? (1 << (b - 1)) : 0;
      if (b > 1) {
        up = (up ? t2 : -t2) <= v;
        stage(__ballot(up), b - 2);
        if (up) idx += 1 << (b - 2);
        for (int k = b - 3; k >= 0; --k) {
          up = t[idx + (1 << k) - 1] <= v;
          stage(__ballot(up), k);
          if (up) idx += 1 << k;
        }
      }
    }
  }
  flush();
}

}  // namespace

void launch_quant(const Geometry& g, int64_t n_units, const float* coef, int64_t ustride,
                  const float* inv_gain, int64_t var_stride, RecordView rec,
                  const uint32_t* plane_off, hipStream_t s) {
  QuantArgs a;
  a.coef = coef;
  a.ustride = ustride;
  a.n_bins = g.n_bins;
  a.total_bits = g.total_bits;
  a.head_dim = g.head_dim;
  a.max_bits = g.max_bits;
  a.inv_gain = inv_gain;
  a.var_stride = var_stride;
  a.plane_off = plane_off;
  a.rec = rec;
  a.rotate = g.rotation == TACT_ROTATION_HADAMARD;
  const int64_t per_block = static_cast<int64_t>(kWave) * kQuantWaves;
  const dim3 grid(static_cast<unsigned>((g.n_bins + per_block - 1) / per_block),
                  static_cast<unsigned>(n_units));
  hipLaunchKernelGGL(k_quant, grid, dim3(kWave * kQuantWaves), 0, s, a);
}

}  // namespace tact
