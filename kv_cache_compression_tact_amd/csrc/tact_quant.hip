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
// step is directly the word of that bit plane.  The coefficients of the next
// eight coded bins are loaded while eight are coded.  The coded bins of a wave
// own one contiguous run of record words (bin by bin, plane by plane, word
// of the plane fastest), so the words are gathered into lanes by their
// position in that run and written up to 64 at a time.
#include <hip/hip_runtime.h>

#include "tact_internal.h"

namespace tact {

#include "codebook_device.h"

// v_writelane_b32 (the compiler's intrinsic): lane `lane` of `old` takes the
// uniform value `v`
__device__ int tact_writelane(int v, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

namespace {

constexpr int kWave = 64;
constexpr int kQuantWaves = 4;
constexpr int kAhead = 8;          // coded bins fetched ahead per wave

struct QuantArgs {
  const float* coef;         // final DCT coefficients, [u][bin][head_dim]
  int64_t ustride;           // elements between units
  int64_t n_bins, total_bits;
  int max_bits;
  RecordView rec;            // header written by the allocation: gains, bits, group index
};

// Codes of one bin of B bits (B >= 1) for its WPP words of 64 channels:
// lane c holds v = coefficient c / gain of each word.  The ballot of step k
// (bit plane k, most significant first) goes to lane base + k * WPP + h of
// the gathered words, which is its place in the record after `base` words.
template <int WPP, int B>
__device__ __forceinline__ void code_bin(const float (&v)[4], const float* __restrict__ s_thr,
                                         int base, int& wlo, int& whi) {
  // the 2^B - 1 sorted thresholds of B bits; the table is symmetric: its
  // middle threshold is 0 and the two next split points are -t2 and +t2
  const float* t = s_thr + ((1 << B) - B - 1);
  float t2 = 0.f;
  if constexpr (B > 1) t2 = t[(3 << (B - 2)) - 1];
  auto stage = [&](bool up, int slot) {
    const uint64_t wd = __ballot(up);
    wlo = tact_writelane(static_cast<int>(static_cast<uint32_t>(wd)), slot, wlo);
    whi = tact_writelane(static_cast<int>(static_cast<uint32_t>(wd >> 32)), slot, whi);
  };
#pragma unroll
  for (int h = 0; h < WPP; ++h) {
    bool up = 0.f <= v[h];
    stage(up, base + (B - 1) * WPP + h);
    if constexpr (B > 1) {
      int idx = up ? (1 << (B - 1)) : 0;
      up = (up ? t2 : -t2) <= v[h];
      stage(up, base + (B - 2) * WPP + h);
      if (up) idx += 1 << (B - 2);
      // q points at threshold idx - 1, the last one known to be <= v
      const float* q = t + idx - 1;
#pragma unroll
      for (int k = B - 3; k >= 0; --k) {
        const float* c = q + (1 << k);
        up = *c <= v[h];
        stage(up, base + k * WPP + h);
        if (up) q = c;
      }
    }
  }
}

// WPP = head_dim / 64 words per bit plane of a bin
template <int WPP>
__global__ __launch_bounds__(kWave * kQuantWaves) void k_quant(QuantArgs a) {
  __shared__ float s_thr[TACT_CODEBOOK_THRESHOLDS];
  for (int j = threadIdx.x; j < TACT_CODEBOOK_THRESHOLDS; j += blockDim.x) s_thr[j] = c_thresholds[j];
  __syncthreads();
  const int lane = threadIdx.x % kWave;
  const int64_t u = blockIdx.y;
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * kQuantWaves + threadIdx.x / kWave) * kWave;
  if (b0 >= a.n_bins) return;
  constexpr int kHeadDim = 64 * WPP;

  // side info of bin b0 + lane, from the record's header: the wave's 64
  // bins are one group of the index, so the first plane of bin b0 + lane is
  // the group's entry plus the widths of the lanes below (a wave scan), and
  // 1/gain is formed from the stored gain as the allocation forms it
  const uint8_t* r = a.rec.base + u * a.rec.stride;
  int bj = 0;
  float ij = 0.f;
  if (b0 + lane < a.n_bins) {
    const int64_t bin = b0 + lane;
    bj = r[a.rec.off_bits + bin];
    const float gn = reinterpret_cast<const float*>(r + a.rec.off_gains)[bin];
    ij = gn > 0.f ? 1.0f / gn : 0.f;
  }
  int incl = bj;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  int pj = static_cast<int>(reinterpret_cast<const uint32_t*>(r + a.rec.off_groups)[b0 / kWave]) + incl - bj;
  if (bj > a.max_bits || static_cast<int64_t>(static_cast<uint32_t>(pj)) + bj > a.total_bits) bj = 0;

  const float* cu = a.coef + u * a.ustride + b0 * kHeadDim + lane;
  uint64_t* words = reinterpret_cast<uint64_t*>(a.rec.base + u * a.rec.stride + a.rec.off_codes);
  // gathered words: lane k holds word first + k of the record
  int wlo = 0, whi = 0;
  int cnt = 0;
  int64_t first = 0;
  auto flush = [&]() {
    if (lane < cnt)
      words[first + lane] = (static_cast<uint64_t>(static_cast<uint32_t>(whi)) << 32) |
                            static_cast<uint32_t>(wlo);
    cnt = 0;
  };

  // coded bins of this wave, lowest first, in groups of kAhead: the
  // coefficients of the next group are in flight while a group is coded
  // (one bin ahead leaves too little in flight to stream the coefficients)
  uint64_t todo = __ballot(bj > 0);
  float nxt[kAhead][4];
  int jn[kAhead];
  int nn = 0;
  auto fetch_group = [&]() {
    nn = 0;
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      jn[i] = todo ? __builtin_ctzll(todo) : 0;
      if (todo) {
        todo &= todo - 1;
        ++nn;
      }
#pragma unroll
      for (int h = 0; h < WPP; ++h) nxt[i][h] = i < nn ? cu[jn[i] * kHeadDim + 64 * h] : 0.f;
    }
  };
  fetch_group();
  while (nn > 0) {
    float cur[kAhead][4];
    int jc[kAhead];
    const int nc = nn;
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      jc[i] = jn[i];
#pragma unroll
      for (int h = 0; h < 4; ++h) cur[i][h] = nxt[i][h];
    }
    fetch_group();
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if (i >= nc) break;
      const int j = jc[i];
      float v[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) v[h] = cur[i][h];
      const int b = __builtin_amdgcn_readlane(bj, j);
      const int64_t w0 = static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(pj, j))) * WPP;
      const float inv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ij), j));
#pragma unroll
      for (int h = 0; h < WPP; ++h) v[h] *= inv;
      // this bin's b * WPP words must follow the gathered ones in the record
      // and fit beside them
      if (cnt > 0 && (w0 != first + cnt || cnt + b * WPP > kWave)) flush();
      if (cnt == 0) first = w0;
      switch (b) {
        case 1: code_bin<WPP, 1>(v, s_thr, cnt, wlo, whi); break;
        case 2: code_bin<WPP, 2>(v, s_thr, cnt, wlo, whi); break;
        case 3: code_bin<WPP, 3>(v, s_thr, cnt, wlo, whi); break;
        case 4: code_bin<WPP, 4>(v, s_thr, cnt, wlo, whi); break;
        case 5: code_bin<WPP, 5>(v, s_thr, cnt, wlo, whi); break;
        case 6: code_bin<WPP, 6>(v, s_thr, cnt, wlo, whi); break;
        case 7: code_bin<WPP, 7>(v, s_thr, cnt, wlo, whi); break;
        default: code_bin<WPP, 8>(v, s_thr, cnt, wlo, whi); break;
      }
      cnt += b * WPP;
    }
  }
  flush();
}

}  // namespace

void launch_quant(const Geometry& g, int64_t n_units, const float* coef, int64_t ustride,
                  RecordView rec, hipStream_t s) {
  QuantArgs a;
  a.coef = coef;
  a.ustride = ustride;
  a.n_bins = g.n_bins;
  a.total_bits = g.total_bits;
  a.max_bits = g.max_bits;
  a.rec = rec;
  const int64_t per_block = static_cast<int64_t>(kWave) * kQuantWaves;
  const dim3 grid(static_cast<unsigned>((g.n_bins + per_block - 1) / per_block),
                  static_cast<unsigned>(n_units));
  const dim3 block(kWave * kQuantWaves);
  if (g.head_dim == 64) hipLaunchKernelGGL(k_quant<1>, grid, block, 0, s, a);
  else if (g.head_dim == 128) hipLaunchKernelGGL(k_quant<2>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_quant<4>, grid, block, 0, s, a);
}

}  // namespace tact
