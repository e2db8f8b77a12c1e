// Coding pass of the TACT-KV codec for gfx950 (page "TACT-KV: Tri-Axis
// Cosine Transform for Compressing Volumetric KV Caches in Medical VLMs",
// section "Methodology in Plain English", stage 4): gain-shape scalar
// quantization of the final DCT coefficients and bit-plane packing.
//
// k_quant streams the coefficient volume once, reading only bins that were
// given bits.  The coefficients arrive already rotated by the quantizer's
// shared rotation when the geometry asks for it (the forward S pass applies
// it), so the value quantized here is coefficient / gain.  One wave owns
// 64 consecutive bins of a unit (lane j reads bin j's bit width, first
// plane and 1/gain) and lists its coded bins in LDS in order, each with its
// coefficient offset, width, first record word and 1/gain.  It then walks
// the list one bin at a time: lane c is channel c of a 64-channel word, so
// a bin's codes for one bit plane are one ballot.  The cell index is found
// most significant bit first (binary search over the sorted thresholds),
// and the ballot of each step is directly the word of that bit plane.  The
// coefficients of the next eight coded bins are loaded while eight are
// coded.  A bin's words (plane by plane, word of the plane fastest) are
// collected in the lanes of their place after the bin's first word and
// written with one store.
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

// Raw buffer access (descriptor word 3 of gfx9 raw buffers): loads past the
// descriptor's byte range return 0 and stores past it are dropped.
constexpr int kBufWord3 = 0x00020000;
// a lane offset past every buffer addressed here (coefficient slices and
// code areas stay below 2^30 bytes)
constexpr int kPastBuffer = 0x7FFFFFF0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufWord3);
}

// Codes of one bin of B bits (B >= 1) for its WPP words of 64 channels:
// lane c holds v = coefficient c / gain of each word.  The ballot of step k
// (bit plane k, most significant first) goes to lane k * WPP + h of the
// bin's words, which is its place in the record after the bin's first word.
template <int WPP, int B>
__device__ __forceinline__ void code_bin(const float (&v)[4], const float* __restrict__ s_thr,
                                         int& wlo, int& whi) {
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
    stage(up, (B - 1) * WPP + h);
    if constexpr (B > 1) {
      int idx = up ? (1 << (B - 1)) : 0;
      up = (up ? t2 : -t2) <= v[h];
      stage(up, (B - 2) * WPP + h);
      if (up) idx += 1 << (B - 2);
      // q points at threshold idx - 1, the last one known to be <= v
      const float* q = t + idx - 1;
#pragma unroll
      for (int k = B - 3; k >= 0; --k) {
        const float* c = q + (1 << k);
        up = *c <= v[h];
        stage(up, k * WPP + h);
        if (up) q = c;
      }
    }
  }
}

// WPP = head_dim / 64 words per bit plane of a bin
template <int WPP>
__global__ __launch_bounds__(kWave * kQuantWaves) void k_quant(QuantArgs a) {
  __shared__ float s_thr[TACT_CODEBOOK_THRESHOLDS];
  // per wave, its coded bins in order: the byte offset of each one's
  // coefficients (kAhead more slots, read past the last coded bin and
  // unused), and {bits, first word, 1/gain}
  __shared__ int s_off[kQuantWaves][kWave + kAhead];
  __shared__ int4 s_side[kQuantWaves][kWave];
  for (int j = threadIdx.x; j < TACT_CODEBOOK_THRESHOLDS; j += blockDim.x) s_thr[j] = c_thresholds[j];
  __syncthreads();
  const int lane = threadIdx.x % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  const int64_t u = blockIdx.y;
  const int64_t b0 = (static_cast<int64_t>(blockIdx.x) * kQuantWaves + wv) * kWave;
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
  const int pj = static_cast<int>(reinterpret_cast<const uint32_t*>(r + a.rec.off_groups)[b0 / kWave]) + incl - bj;
  if (bj > a.max_bits || static_cast<int64_t>(static_cast<uint32_t>(pj)) + bj > a.total_bits) bj = 0;

  // the coded bins, listed in order by their rank among the wave's coded bins
  const uint64_t coded = __ballot(bj > 0);
  const int n = __builtin_popcountll(coded);
  if (n == 0) return;
  if (bj > 0) {
    const int rank = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<uint32_t>(coded >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(coded), 0u)));
    s_off[wv][rank] = lane * kHeadDim * 4;
    s_side[wv][rank] = int4{bj, pj * WPP, __float_as_int(ij), 0};
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // the wave's coefficients (64 bins, fewer in the last wave of a unit) and
  // the unit's code words, as buffers
  const int64_t nb = a.n_bins - b0 < kWave ? a.n_bins - b0 : kWave;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.coef + u * a.ustride + b0 * kHeadDim, nb * kHeadDim * 4);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(a.rec.base + u * a.rec.stride + a.rec.off_codes, a.total_bits * WPP * 8);

  // coded bins in groups of kAhead: the coefficients of the next group are
  // in flight while a group is coded (one bin ahead leaves too little in
  // flight to stream the coefficients).  Every group issues the same loads
  // and stores: ranks past the last coded bin use an offset past the
  // buffer, so the wait for a group's loads counts the stores after them.
  float nxt[kAhead][4];
  auto fetch_group = [&](int r0) {
    int so[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) so[i] = s_off[wv][r0 + i];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int off = r0 + i < n ? so[i] + 4 * lane : kPastBuffer;
#pragma unroll
      for (int h = 0; h < WPP; ++h)
        nxt[i][h] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, off, 256 * h, 0));
    }
  };
  fetch_group(0);
  for (int r0 = 0; r0 < n; r0 += kAhead) {
    float cur[kAhead][4];
#pragma unroll
    for (int i = 0; i < kAhead; ++i)
#pragma unroll
      for (int h = 0; h < WPP; ++h) cur[i][h] = nxt[i][h];
    // (the last group fetches past the list: offsets past the buffer)
    fetch_group(r0 + kAhead < kWave ? r0 + kAhead : kWave);
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      int wlo = 0, whi = 0;
      int off = kPastBuffer;
      if (r0 + i < n) {
        const int4 sc = s_side[wv][r0 + i];
        const int b = __builtin_amdgcn_readfirstlane(sc.x);
        const float inv = __int_as_float(sc.z);
        float v[4];
#pragma unroll
        for (int h = 0; h < WPP; ++h) v[h] = cur[i][h] * inv;
        switch (b) {
          case 1: code_bin<WPP, 1>(v, s_thr, wlo, whi); break;
          case 2: code_bin<WPP, 2>(v, s_thr, wlo, whi); break;
          case 3: code_bin<WPP, 3>(v, s_thr, wlo, whi); break;
          case 4: code_bin<WPP, 4>(v, s_thr, wlo, whi); break;
          case 5: code_bin<WPP, 5>(v, s_thr, wlo, whi); break;
          case 6: code_bin<WPP, 6>(v, s_thr, wlo, whi); break;
          case 7: code_bin<WPP, 7>(v, s_thr, wlo, whi); break;
          default: code_bin<WPP, 8>(v, s_thr, wlo, whi); break;
        }
        // the bin's b * WPP words: lane k * WPP + h is word first + k * WPP + h
        if (lane < b * WPP) off = (sc.y + lane) * 8;
      }
      __builtin_amdgcn_raw_buffer_store_b64(
          __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))),
                             uint2{static_cast<uint32_t>(wlo), static_cast<uint32_t>(whi)}),
          rw, off, 0, 0);
    }
  }
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
