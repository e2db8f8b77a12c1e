// Coding pass of the TACT-KV codec for gfx950 (page "TACT-KV: Tri-Axis
// Cosine Transform for Compressing Volumetric KV Caches in Medical VLMs",
// section "Methodology in Plain English", stage 4): gain-shape scalar
// quantization of the final DCT coefficients and bit-plane packing.
//
// k_quant streams the coefficient volume once, reading only bins that were
// given bits.  The coefficients arrive already rotated by the quantizer's
// shared rotation when the geometry asks for it (the forward S pass applies
// it), so the value quantized here is coefficient / gain.  One wave owns 64 consecutive bins of a unit (lane j holds
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

struct QuantArgs {
  const float* coef;         // final DCT coefficients, [u][bin][head_dim]
  int64_t ustride;           // elements between units
  int64_t n_bins, total_bits;
  int head_dim, max_bits;
  const float* inv_gain;     // fp32 1/gain per bin (0 for gain 0)
  int64_t var_stride;        // floats per unit in inv_gain
  const uint32_t* plane_off; // first bit plane of each bin, [u][bin]
  RecordView rec;
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
      const float v = cur[h] * inv;
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
  const int64_t per_block = static_cast<int64_t>(kWave) * kQuantWaves;
  const dim3 grid(static_cast<unsigned>((g.n_bins + per_block - 1) / per_block),
                  static_cast<unsigned>(n_units));
  hipLaunchKernelGGL(k_quant, grid, dim3(kWave * kQuantWaves), 0, s, a);
}

}  // namespace tact
