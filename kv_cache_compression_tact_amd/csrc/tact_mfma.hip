// MFMA path of the TACT-KV codec for gfx950 (page "TACT-KV: Tri-Axis Cosine
// Transform for Compressing Volumetric KV Caches in Medical VLMs", section
// "Methodology in Plain English", stages 2-4 and the decoding paragraph).
//
// k_axis: one axis of the separable DCT as dense matrix products on the
// matrix cores.  The axis of length N is the contraction (K) dimension,
// padded to 16/32/64; the columns are 16 consecutive elements of the
// contiguous trailing dimensions (one 64-byte run per 16 lanes).  Products
// keep fp32 accuracy with split fp16 operands: the DCT matrix, scaled by
// 2^12, is C_hi + C_lo; every column is scaled by a power of two that puts
// its largest magnitude in [2^13, 2^14) and split x_hi + x_lo, so each
// operand carries ~22 significant bits (|x - x_hi - x_lo| <= 2^-22 |x| plus
// a floor 2^-38 below the column maximum).  bf16 inputs are exact in fp16
// and need C_hi*x + C_lo*x; fp32 inputs add C_hi*x_lo.  Accumulation is fp32
// inside the MFMA; the power-of-two scales are undone exactly on output.
//   prologues:  bf16 / fp32 loads, or dequantization straight from a record
//               (first inverse axis);
//   epilogues:  fp32 / bf16 stores, per-bin variance (last forward axis,
//               statistics pass), or quantization + bit-plane packing (last
//               forward axis, coding pass).
//
// k_alloc_*: reverse water-filling as an exact radix selection of the T-th
// largest marginal gain (3 histogram sweeps instead of a long bisection), on
// several workgroups per unit, then the index-ordered tie rule, record
// header and per-bin plane offsets.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tact_internal.h"

namespace tact {

#include "codebook_device.h"

namespace {

constexpr int kWave = 64;

#include "tact_mfma_ops.h"

// the Lloyd-Max levels are scaled the same way when they are a matrix
// operand

constexpr float kLevelScale = 2048.0f;

// ---------------------------------------------------------------------------
// DCT-II matrices of the three axes, fp32, zero padded to 64 x 64:
// tab[a][k][n] = a_k cos(pi (2n+1) k / 2N_a), a_0 = sqrt(1/N), a_k = sqrt(2/N).
// Axis a takes the identity instead when bit a of `identity` is set (the S
// axis for no-transform coding; every axis for the decoding stage call, which
// then returns the dequantized coefficients).
// ---------------------------------------------------------------------------
__global__ void k_dct_tables(float* __restrict__ tab, int n0, int n1, int n2, int identity) {
  const int a = blockIdx.x;
  const int N = a == 0 ? n0 : (a == 1 ? n1 : n2);
  for (int e = threadIdx.x; e < 64 * 64; e += blockDim.x) {
    const int k = e / 64, n = e % 64;
    float v = 0.f;
    if (k < N && n < N) {
      if ((identity >> a) & 1) {
        v = k == n ? 1.f : 0.f;
      } else {
        const double al = (k == 0) ? sqrt(1.0 / N) : sqrt(2.0 / N);
        v = static_cast<float>(al * cospi((2.0 * n + 1.0) * k / (2.0 * N)));
      }
    }
    tab[a * 4096 + e] = v;
  }
}


__device__ __forceinline__ uint16_t bf16_rne_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// The shared rotation of the quantizer (stage 4), R = H_64 diag(s) / 8 on
// every 64-channel block of a bin (tact_rotation.h).  In the fragments the 6
// channel bits split into 4 lane bits (lanes of a 16-lane row) and 2
// register bits (4 values per lane).
// ---------------------------------------------------------------------------
#include "tact_rotation.h"
#include "tact_lane_ops.h"
#include "tact_bitplanes.h"

// Raw buffer access (descriptor word 3 of gfx9 raw buffers): loads past
// the descriptor's byte range return 0 and stores past it are dropped, so
// padded rows need no branch.  voff is per lane, soff uniform.
constexpr int kBufWord3 = 0x00020000;
// a lane offset past every buffer the kernels address: a unit's padded fp32
// volume is at most 2^30 bytes, so descriptor ranges stay below it and a
// uniform offset added to it does not wrap past 2^32
constexpr int kPastBuffer = 0x7FFFFFF0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufWord3);
}
__device__ __forceinline__ float4 buf_ld4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// A store of more than 8 bytes may read its data registers after it
// issues; a VALU write to those registers in the very next instruction can
// reach memory instead.  Every 128-bit store is followed by one wait state.
__device__ __forceinline__ void store_gap() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 0");
  __builtin_amdgcn_sched_barrier(0);
}
// AUX: cache policy bits of the store (2 = nt, streaming: data not reused
// soon)
template <int AUX = 0>
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, int voff, int soff, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint32_t __attribute__((ext_vector_type(4))), v),
                                         r, voff, soff, AUX);
  store_gap();
}

// 128-bit LDS access at a float offset that is a multiple of 4
__device__ __forceinline__ float4 lds_ld4(const float* p) {
  return *static_cast<const float4*>(__builtin_assume_aligned(p, 16));
}
__device__ __forceinline__ void lds_st4(float* p, float4 v) {
  *static_cast<float4*>(__builtin_assume_aligned(p, 16)) = v;
}

// The same for 8 channels per lane (channel 8 t + i): in-register
// butterflies over the 3 register bits, then lanes ^ 1, ^ 2, ^ 4; the
// result is parity8 * (H_64 x).
__device__ __forceinline__ void wht64_r8(float (&y)[8], const LaneWht& w) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const float a0 = y[i], a1 = y[i + h];
        y[i] = a0 + a1;
        y[i + h] = a0 - a1;
      }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float x = y[q];
    x = fmaf(lane_xor1(x), w.sg[0], x);
    x = fmaf(lane_xor2(x), w.sg[1], x);
    x = fmaf(lane_xor4(x), w.sg[2], x);
    y[q] = x;
  }
}

// Number of the 2^b - 1 ascending thresholds (LDS copy) that are <= u.
__device__ __forceinline__ int cell_index_lds(const float* thr, float u, int b) {
  const float* t = thr + ((1 << b) - b - 1);
  int pos = 0;
  for (int step = 1 << (b - 1); step >= 1; step >>= 1)
    if (t[pos + step - 1] <= u) pos += step;
  return pos;
}

enum Pro { PRO_BF16 = 0, PRO_F32 = 1, PRO_DEQUANT = 2 };
enum Epi { EPI_F32 = 0, EPI_BF16 = 1, EPI_STATS = 2, EPI_QUANT = 3 };

struct AxisArgs {
  const void* in;
  int64_t in_ustride;        // elements between units
  void* out;
  int64_t out_ustride;
  const float* tab;          // 64 x 64 matrix of this axis
  int inverse;               // multiply by C^T instead of C
  int N;                     // axis length
  int64_t outer, inner;      // columns: outer x inner, inner contiguous
  int64_t n_units;
  // bins (epilogues / dequant prologue)
  int head_dim, kv_heads;
  int64_t C;                 // kv_heads * head_dim
  int64_t n_bins;
  int64_t total_bits;
  int max_bits;
  float* var;                // EPI_STATS: var[u * var_stride + bin]
  const float* inv_gain;     // EPI_QUANT: fp32 1/gain per bin (0 for gain 0), same stride
  int64_t var_stride;
  RecordView rec;            // EPI_QUANT, PRO_DEQUANT
  const uint32_t* plane_off; // per-bin first plane, u * n_bins + bin
  int rotate;                // EPI_QUANT, PRO_DEQUANT: apply the shared rotation
  int rot_in;                // PRO_F32 plain pass (4 channels per lane): apply the
                             // inverse rotation R^T to the input rows
  int rot_out;               // EPI_F32 plain pass: apply the rotation R to the
                             // output rows
  int quant;                 // EPI_QUANT, PRO_DEQUANT: tact_params.quantizer; for
                             // the uniform and NormalFloat tables EPI_QUANT
                             // takes each bin's gain as its largest |value|
                             // and writes it into the record
};


// Column layout of one wave: TPW tiles of 16 columns.
//   interleaved (plain passes): tile i holds columns c0 + TPW*t + i, so each
//     lane loads and stores TPW consecutive elements as one vector;
//   contiguous (variance / quantize passes): tile i holds c0 + 16*i + t, so
//     a tile is 16 consecutive channels of one head.
template <int TPW, bool INTL>
__device__ __forceinline__ int64_t col_of(int64_t c0, int i, int t) {
  return INTL ? c0 + TPW * t + i : c0 + 16 * i + t;
}

// Grid: x = groups of 4 waves along the columns (each wave loops over
// column groups), y = outer index o, z = unit.  One wave: TPW tiles.
template <int NP, int PRO, int EPI, int TPW>
__global__ __launch_bounds__(256) void k_axis(AxisArgs a) {
  static_assert(PRO != PRO_DEQUANT || TPW == 4, "dequant reads one 64-channel word per plane");
  constexpr bool INTL = (EPI == EPI_F32 || EPI == EPI_BF16);
  static_assert(!INTL || TPW == 4 || TPW == 8, "vector width");
  static_assert(!INTL || PRO != PRO_F32 || TPW == 4, "fp32 rows load 4 floats");
  using F = Frag<NP>;
  using vec = typename F::vec;
  const int lane = threadIdx.x % kWave;
  const int t = lane % 16, g = lane / 16;
  const int64_t u = blockIdx.z;
  const int64_t o = blockIdx.y;
  const int64_t groups = a.inner / (16 * TPW);
  __shared__ float s_levels[(PRO == PRO_DEQUANT) ? TACT_CODEBOOK_LEVELS : 1];
  __shared__ float s_thr[(EPI == EPI_QUANT) ? TACT_CODEBOOK_THRESHOLDS : 1];
  // bin-major staging of one wave's coefficients: quantize (rows = output
  // frequencies, 16 * TPW channels) or dequantize (rows = input frequencies,
  // 64 channels); rows padded by 4 floats to spread LDS banks
  constexpr int ZROW = 16 * TPW + 4;
  // rows staged at once: at most 32 for the widest heads (LDS budget)
  constexpr int ZROWS = (TPW == 16 && NP > 32) ? 32 : NP;
  __shared__ __attribute__((aligned(16))) float s_z[(EPI == EPI_QUANT) ? 4 * ZROWS * ZROW : 1];
  __shared__ __attribute__((aligned(16))) float s_d[(PRO == PRO_DEQUANT) ? 4 * NP * 68 : 1];
  if constexpr (PRO == PRO_DEQUANT || EPI == EPI_QUANT) {
    if constexpr (PRO == PRO_DEQUANT)
      for (int j = threadIdx.x; j < TACT_CODEBOOK_LEVELS; j += blockDim.x) s_levels[j] = c_levels_q[a.quant][j];
    if constexpr (EPI == EPI_QUANT)
      for (int j = threadIdx.x; j < TACT_CODEBOOK_THRESHOLDS; j += blockDim.x) s_thr[j] = c_thresholds_q[a.quant][j];
    __syncthreads();
  }
  const int N = a.N;
  // the shared rotation: lane butterflies and per-tile post factors
  // (dequantize: channel 4t + i; quantize: channel 16 (i % 4) + t)
  const LaneWht wl(lane);
  // per-tile output factors of the rotation: signs s_j and 1/8 folded into
  // the output scale
  float rpost[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) rpost[i] = 1.f;
  const bool rot = (PRO == PRO_DEQUANT || EPI == EPI_QUANT) && a.rotate;
  // inverse rotation of plain fp32 rows: channel 4t + i of a 64-column word
  const bool rot_in = INTL && PRO == PRO_F32 && TPW == 4 && a.rot_in;
  // rotation of plain fp32 output rows, channel TPW t + i: R = H diag(s) / 8
  // with s on the input side (commutes with the contraction), H after it
  const bool rot_out = INTL && EPI == EPI_F32 && a.rot_out;
  if (rot || rot_in) {
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      rpost[i] = (PRO == PRO_DEQUANT || rot_in) ? 0.125f * wl.parity * rotation_sign(4 * t + (i % 4))
                                                : rotation_sign(16 * (i % 4) + t);
  } else if (rot_out) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) rpost[i] = rotation_sign((TPW * t + i) % 64);
  }

  // A fragments (the DCT matrix scaled by 2^12, or its transpose), hi / lo
  vec ahi[F::MT][F::KSTEPS], alo[F::MT][F::KSTEPS];
#pragma unroll
  for (int m = 0; m < F::MT; ++m)
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
      for (int v = 0; v < F::KV; ++v) {
        const int row = 16 * m + t;
        const int col = ks * F::KPER + F::KV * g + v;
        const float c = kMatScale * (a.inverse ? a.tab[col * 64 + row] : a.tab[row * 64 + col]);
        _Float16 h, l;
        split2(c, h, l);
        ahi[m][ks][v] = h;
        alo[m][ks][v] = l;
      }

  const int64_t col_stride = a.inner;                 // element step along the axis
  const int64_t obase = o * static_cast<int64_t>(N) * a.inner;
  const int64_t bins_per_k = (a.inner / a.C) * a.kv_heads;   // bin step per frequency

  // Plain passes (interleaved columns): rows n of this (unit, o) through a
  // buffer of N rows, so rows n >= N read 0 and output rows k >= N are
  // dropped; byte offsets, padded rows included, fit 31 bits (a unit's
  // padded fp32 volume is at most 2^30 bytes).
  // The next column group's rows are fetched while this one is computed.
  constexpr bool PF = INTL && PRO != PRO_DEQUANT;
  constexpr int ES_IN = (PRO == PRO_BF16) ? 2 : 4;
  constexpr int ES_OUT = (EPI == EPI_BF16) ? 2 : 4;
  const int row_in = static_cast<int>(a.inner) * ES_IN;
  const int row_out = static_cast<int>(a.inner) * ES_OUT;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(
      PF ? static_cast<const char*>(a.in) + (u * a.in_ustride + obase) * ES_IN : nullptr,
      PF ? static_cast<int64_t>(row_in) * N : 0);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(
      INTL ? static_cast<const char*>(a.out) + (u * a.out_ustride + obase) * ES_OUT : nullptr,
      INTL ? static_cast<int64_t>(row_out) * N : 0);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  auto fetch = [&](int64_t grp_, u32x4 (&r)[F::KSTEPS][F::KV]) {
    const int vo = F::KV * g * row_in + static_cast<int>(grp_ * (16 * TPW) + TPW * t) * ES_IN;
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
      for (int v = 0; v < F::KV; ++v) {
        const int so = (ks * F::KPER + v) * row_in;
        if constexpr (TPW * ES_IN == 16) {
          r[ks][v] = __builtin_amdgcn_raw_buffer_load_b128(rin, vo, so, 0);
        } else {
          const auto q = __builtin_amdgcn_raw_buffer_load_b64(rin, vo, so, 0);
          r[ks][v] = u32x4{q[0], q[1], 0u, 0u};
        }
      }
  };
  const int64_t grp_step = static_cast<int64_t>(gridDim.x) * 4;
  u32x4 cur[PF ? F::KSTEPS : 1][PF ? F::KV : 1];
  if constexpr (PF) {
    const int64_t g0 = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
    if (g0 < groups) fetch(g0, cur);
  }

  for (int64_t grp = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave; grp < groups;
       grp += grp_step) {
    const int64_t c0 = grp * (16 * TPW);
    u32x4 nxt[PF ? F::KSTEPS : 1][PF ? F::KV : 1];
    if constexpr (PF) {
      if (grp + grp_step < groups) {
        fetch(grp + grp_step, nxt);
      } else {
#pragma unroll
        for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
          for (int v = 0; v < F::KV; ++v) nxt[ks][v] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    // bin of frequency k at this column start: bin0 + k * bins_per_k
    const int64_t bin0 =
        (o * N * (a.inner / a.C) + c0 / a.C) * a.kv_heads + (c0 % a.C) / a.head_dim;

    f32x4 acc[TPW][F::MT];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int m = 0; m < F::MT; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    float xv[PF ? 1 : TPW][F::KSTEPS][F::KV];
    if constexpr (PRO == PRO_DEQUANT) {
      // first inverse axis: coefficients come from the record
      const uint8_t* r = a.rec.base + u * a.rec.stride;
      const uint8_t* bits = r + a.rec.off_bits;
      const float* gains = reinterpret_cast<const float*>(r + a.rec.off_gains);
      const uint64_t* words = reinterpret_cast<const uint64_t*>(r + a.rec.off_codes);
      const uint32_t* poff = a.plane_off + u * a.n_bins;
      const int wpp = a.head_dim / 64;
      const int ch0 = static_cast<int>(c0 % a.head_dim);   // multiple of 64
      // decode one bin at a time (its bit width is uniform over the wave):
      // lane j is channel ch0 + j of the bin's 64-bit code words
      float* dt = s_d + (threadIdx.x / kWave) * NP * 68;
      // lane j fetches bin j's bits, gain, first plane and code words (all
      // loads in flight together); the decode loop broadcasts them
      int bj = 0;
      float gj = 0.f;
      uint32_t wlo[8], whi[8];
      {
        int64_t pj = 0;
        if (lane < N) {
          const int64_t bin = bin0 + lane * bins_per_k;
          bj = bits[bin];
          pj = poff[bin];
          gj = gains[bin];
          if (bj > a.max_bits || pj + bj > a.total_bits) bj = 0;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          uint64_t w = 0;
          if (q < bj) w = words[(pj + q) * wpp + ch0 / 64];
          wlo[q] = static_cast<uint32_t>(w);
          whi[q] = static_cast<uint32_t>(w >> 32);
        }
      }
      for (int n = 0; n < N; ++n) {
        const int b = __builtin_amdgcn_readlane(bj, n);
        float x = 0.f;
        if (b > 0) {
          int code = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (q < b) {
              const uint32_t lo = __builtin_amdgcn_readlane(wlo[q], n);
              const uint32_t hi = __builtin_amdgcn_readlane(whi[q], n);
              const uint32_t wd = lane < 32 ? lo : hi;
              code |= static_cast<int>((wd >> (lane & 31)) & 1u) << q;
            }
          }
          x = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gj), n)) *
              s_levels[(1 << b) - 2 + code];
        }
        dt[n * 68 + lane] = x;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
        for (int v = 0; v < F::KV; ++v) {
          const int n = ks * F::KPER + F::KV * g + v;
          float4 q = float4{0.f, 0.f, 0.f, 0.f};
          if (n < N) q = lds_ld4(dt + n * 68 + TPW * t);
          xv[0][ks][v] = q.x;
          xv[1][ks][v] = q.y;
          xv[2][ks][v] = q.z;
          xv[3][ks][v] = q.w;
        }
      // R^T = diag(s) H / 8: H here, the rest with the output scale
      if (rot) {
#pragma unroll
        for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
          for (int v = 0; v < F::KV; ++v)
            wht64(xv[0][ks][v], xv[1][ks][v], xv[2][ks][v], xv[3][ks][v], wl);
      }
    } else if constexpr (INTL) {
      // rows come from the prefetch registers (cur), one tile at a time;
      // R^T = diag(s) H / 8 on fp32 rows: H here, the rest with the output
      // scale
      if constexpr (PRO == PRO_F32 && TPW == 4) {
        if (rot_in) {
#pragma unroll
          for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
            for (int v = 0; v < F::KV; ++v) {
              float y0 = __uint_as_float(cur[ks][v][0]), y1 = __uint_as_float(cur[ks][v][1]);
              float y2 = __uint_as_float(cur[ks][v][2]), y3 = __uint_as_float(cur[ks][v][3]);
              wht64(y0, y1, y2, y3, wl);
              cur[ks][v] = u32x4{__float_as_uint(y0), __float_as_uint(y1), __float_as_uint(y2),
                                 __float_as_uint(y3)};
            }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int64_t c = c0 + 16 * i + t;
#pragma unroll
        for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
          for (int v = 0; v < F::KV; ++v) {
            const int n = ks * F::KPER + F::KV * g + v;
            float x = 0.f;
            if (n < N) {
              const int64_t idx = u * a.in_ustride + obase + n * col_stride + c;
              if constexpr (PRO == PRO_BF16)
                x = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.in)[idx]) << 16);
              else
                x = static_cast<const float*>(a.in)[idx];
            }
            xv[i][ks][v] = x;
          }
      }
    }

#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      // tile i: column c0 + TPW t + i (interleaved) or c0 + 16 i + t
      float xi[F::KSTEPS][F::KV];
#pragma unroll
      for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
        for (int v = 0; v < F::KV; ++v) {
          if constexpr (PF && PRO == PRO_BF16) {
            const uint32_t w = cur[ks][v][i / 2];
            xi[ks][v] = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
          } else if constexpr (PF) {
            xi[ks][v] = __uint_as_float(cur[ks][v][i]);
          } else {
            xi[ks][v] = xv[i][ks][v];
          }
        }
      float mx = 0.f;
#pragma unroll
      for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
        for (int v = 0; v < F::KV; ++v) mx = fmaxf(mx, fabsf(xi[ks][v]));
      mx = column_max(mx);
      // scale 2^(14 - e) puts the column maximum m = f 2^e in [2^13, 2^14);
      // output scale: 2^-12 (matrix) * 2^(e - 14) (column)
      int e = 0;
      if (mx > 0.f) frexpf(mx, &e);
      const float sc = ldexpf(1.0f, 14 - e);
      const float unscale = ldexpf(1.0f, e - 26) * rpost[i];
#pragma unroll
      for (int ks = 0; ks < F::KSTEPS; ++ks) {
        uint32_t hw[F::KV / 2], lw[F::KV / 2];
#pragma unroll
        for (int v = 0; v < F::KV; v += 2) {
          hw[v / 2] = split_hi_pair(xi[ks][v], sc, xi[ks][v + 1], sc);
          // a scaled bf16 input is exact in fp16 down to 2^-14, 2^27 below
          // the column maximum: its x_lo term is negligible and skipped
          if constexpr (PRO != PRO_BF16) lw[v / 2] = split_lo_pair(xi[ks][v], sc, xi[ks][v + 1], sc, hw[v / 2]);
        }
        const vec bhi = pairs_to_vec<NP>(hw);
#pragma unroll
        for (int m = 0; m < F::MT; ++m) {
          acc[i][m] = mfma<NP>(ahi[m][ks], bhi, acc[i][m]);
          acc[i][m] = mfma<NP>(alo[m][ks], bhi, acc[i][m]);
        }
        if constexpr (PRO != PRO_BF16) {
          const vec blo = pairs_to_vec<NP>(lw);
#pragma unroll
          for (int m = 0; m < F::MT; ++m) acc[i][m] = mfma<NP>(ahi[m][ks], blo, acc[i][m]);
        }
      }
#pragma unroll
      for (int m = 0; m < F::MT; ++m) acc[i][m] *= unscale;
    }

    // ---- epilogues ---------------------------------------------------------
    if constexpr (EPI == EPI_F32 && INTL) {
      if (rot_out) {
        // H_64 on channel TPW t + i: 4 channels per lane -> 2 register bits
        // and 4 lane bits; 8 per lane -> 3 register bits and 3 lane bits
        const float post = 0.125f * (TPW == 8 ? wl.parity8 : wl.parity);
#pragma unroll
        for (int m = 0; m < F::MT; ++m)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            if constexpr (TPW == 8) {
              float y[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) y[i] = acc[i][m][rr];
              wht64_r8(y, wl);
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[i][m][rr] = y[i] * post;
            } else {
              float y0 = acc[0][m][rr], y1 = acc[1][m][rr], y2 = acc[2][m][rr], y3 = acc[3][m][rr];
              wht64(y0, y1, y2, y3, wl);
              acc[0][m][rr] = y0 * post;
              acc[1][m][rr] = y1 * post;
              acc[2][m][rr] = y2 * post;
              acc[3][m][rr] = y3 * post;
            }
          }
      }
    }
    if constexpr (EPI == EPI_F32 || EPI == EPI_BF16) {
      // output row k = 16 m + 4 g + rr; rows k >= N fall past the buffer
      const int vo = 4 * g * row_out + static_cast<int>(c0 + TPW * t) * ES_OUT;
#pragma unroll
      for (int m = 0; m < F::MT; ++m)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int so = (16 * m + rr) * row_out;
          if constexpr (EPI == EPI_F32) {
#pragma unroll
            for (int i = 0; i < TPW; i += 4)
              buf_st4(rout, vo + 4 * i, so,
                      float4{acc[i][m][rr], acc[i + 1][m][rr], acc[i + 2][m][rr], acc[i + 3][m][rr]});
          } else {
            uint32_t w[TPW / 2];
#pragma unroll
            for (int i = 0; i < TPW; i += 2)
              w[i / 2] = bf16_rne_bits(acc[i][m][rr]) |
                         (static_cast<uint32_t>(bf16_rne_bits(acc[i + 1][m][rr])) << 16);
            if constexpr (TPW == 8) {
              __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rout, vo, so, 0);
              store_gap();
            } else
              __builtin_amdgcn_raw_buffer_store_b64(
                  __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))), uint2{w[0], w[1]}),
                  rout, vo, so, 0);
          }
        }
    } else if constexpr (EPI == EPI_STATS) {
      // one wave covers the head_dim channels of one head: TPW == head_dim / 16;
      // raw sum of squares (the allocation applies 1/head_dim)
#pragma unroll
      for (int m = 0; m < F::MT; ++m)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float sq = 0.f;
#pragma unroll
          for (int i = 0; i < TPW; ++i) sq = fmaf(acc[i][m][rr], acc[i][m][rr], sq);
          sq = row_sum16(sq);
          const int k = 16 * m + 4 * g + rr;
          if (t == 0 && k < N) a.var[u * a.var_stride + bin0 + k * bins_per_k] = sq;
        }
    } else {  // EPI_QUANT
      uint8_t* r = a.rec.base + u * a.rec.stride;
      const uint8_t* bits = r + a.rec.off_bits;
      uint64_t* words = reinterpret_cast<uint64_t*>(r + a.rec.off_codes);
      const uint32_t* poff = a.plane_off + u * a.n_bins;
      const float* invg = a.inv_gain + u * a.var_stride;
      float* gains = reinterpret_cast<float*>(r + a.rec.off_gains);
      const bool absmax = a.quant != 0;
      constexpr int HALVES = TPW / 4;                  // 64-channel words per plane
      float* zt = s_z + (threadIdx.x / kWave) * ZROWS * ZROW;
      if (rot) {
        // R = H diag(s) / 8 on each 64-channel word (the signs came with
        // the output scale): channel 16 i' + t of word h is acc[4h + i']
        const float post = 0.125f * wl.parity;
#pragma unroll
        for (int h = 0; h < HALVES; ++h)
#pragma unroll
          for (int m = 0; m < F::MT; ++m)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              float y0 = acc[4 * h][m][rr], y1 = acc[4 * h + 1][m][rr];
              float y2 = acc[4 * h + 2][m][rr], y3 = acc[4 * h + 3][m][rr];
              wht64(y0, y1, y2, y3, wl);
              acc[4 * h][m][rr] = y0 * post;
              acc[4 * h + 1][m][rr] = y1 * post;
              acc[4 * h + 2][m][rr] = y2 * post;
              acc[4 * h + 3][m][rr] = y3 * post;
            }
      }
#pragma unroll
      for (int s0 = 0; s0 < NP; s0 += ZROWS) {
        // bin-major staging: row k - s0 holds the head's 16 * TPW coefficients
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
          for (int m = s0 / 16; m < (s0 + ZROWS) / 16; ++m)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              zt[(16 * m + 4 * g + rr - s0) * ZROW + 16 * i + t] = acc[i][m][rr];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // one bin at a time: uniform bit width, lane j = channel j of a word;
        // lane j prefetches the bits / first plane / reciprocal gain of bin j
        const int kend = (s0 + ZROWS < N) ? s0 + ZROWS : N;
        int bj = 0;
        int pjlo = 0;
        float ij = 0.f;
        if (s0 + lane < kend) {
          const int64_t bin = bin0 + (s0 + lane) * bins_per_k;
          bj = bits[bin];
          const int64_t pj = poff[bin];
          if (bj > a.max_bits || pj + bj > a.total_bits) bj = 0;
          pjlo = static_cast<int>(pj);
          ij = invg[bin];
        }
        for (int k = s0; k < kend; ++k) {
          const int b = __builtin_amdgcn_readlane(bj, k - s0);
          float inv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ij), k - s0));
          if (absmax) {
            // gain of every bin = largest |value| of its (rotated) vector
            float mx = 0.f;
#pragma unroll
            for (int h = 0; h < HALVES; ++h) mx = fmaxf(mx, fabsf(zt[(k - s0) * ZROW + 64 * h + lane]));
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
            if (lane == 0) gains[bin0 + k * bins_per_k] = mx;
            inv = mx > 0.f ? 1.0f / mx : 0.f;
          }
          if (b == 0) continue;
          const int64_t p0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(pjlo, k - s0));
#pragma unroll
          for (int h = 0; h < HALVES; ++h) {
            const int code = cell_index_lds(s_thr, zt[(k - s0) * ZROW + 64 * h + lane] * inv, b);
            for (int q = 0; q < b; ++q) {
              const uint64_t word = __ballot((code >> q) & 1);
              if (lane == 0) words[(p0 + q) * HALVES + h] = word;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
    if constexpr (PF) {
#pragma unroll
      for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
        for (int v = 0; v < F::KV; ++v) cur[ks][v] = nxt[ks][v];
    }
  }
}

// ---------------------------------------------------------------------------
// k_plane: the H and W axes of one (unit, slice s, 64-channel slab) at a
// time in one block.  The H x W x 64 plane lives in LDS between the two
// contractions, so the fp32 volume crosses HBM once per direction instead
// of twice.
//   forward (MODE_STATS): H from global memory into LDS, then W from LDS;
//     the final coefficients go back over the input (in place) together
//     with per-slab partial sums of squares of every bin;
//   inverse (MODE_DEQUANT): decode + inverse W into LDS, then inverse H
//     to global memory.
// A wave owns whole rows of the plane (w columns in the first contraction,
// kh rows in the second), so its LDS rows need no barrier beyond the one
// between the two contractions.
// ---------------------------------------------------------------------------
enum PlaneMode { MODE_STATS = 0, MODE_DEQUANT = 2 };

struct PlaneArgs {
  const float* in;           // forward: the volume after the S axis; unused inverse
  float* out;                // forward: the coefficients (may equal in);
                             // inverse: the volume before the inverse S axis
  int64_t ustride;           // elements between units of in / out
  const float* tab;          // tab[3][64][64]
  int S, H, W;
  int64_t C;                 // kv_heads * head_dim
  int head_dim, kv_heads;
  int64_t n_bins, total_bits;
  int max_bits;
  float* var_part;           // MODE_STATS: raw sums of squares per plane,
                             // [u][slab][s][kh][kw] (slab = 64-channel word)
  int parts;                 // head_dim / 64
  int64_t var_stride;        // floats per unit in var_part
  RecordView rec;
  const uint32_t* plane_off;
  int64_t n_units;
};


// acc[i][m] = post[i] * A * B for 4 interleaved column tiles whose K values
// are xv[i][ks][v]; per-column power-of-two scaling, 3-term split products.
template <int NP>
__device__ __forceinline__ void contract4(const typename Frag<NP>::vec (&ahi)[Frag<NP>::MT][Frag<NP>::KSTEPS],
                                          const typename Frag<NP>::vec (&alo)[Frag<NP>::MT][Frag<NP>::KSTEPS],
                                          float (&xv)[4][Frag<NP>::KSTEPS][Frag<NP>::KV],
                                          f32x4 (&acc)[4][Frag<NP>::MT], const float (&post)[4]) {
  using F = Frag<NP>;
  using vec = typename F::vec;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 0; m < F::MT; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mx = 0.f;
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
      for (int v = 0; v < F::KV; ++v) mx = fmaxf(mx, fabsf(xv[i][ks][v]));
    mx = column_max(mx);
    int e = 0;
    if (mx > 0.f) frexpf(mx, &e);
    const float sc = ldexpf(1.0f, 14 - e);
    const float unscale = ldexpf(1.0f, e - 26) * post[i];
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks) {
      uint32_t hw[F::KV / 2], lw[F::KV / 2];
#pragma unroll
      for (int v = 0; v < F::KV; v += 2) {
        hw[v / 2] = split_hi_pair(xv[i][ks][v], sc, xv[i][ks][v + 1], sc);
        lw[v / 2] = split_lo_pair(xv[i][ks][v], sc, xv[i][ks][v + 1], sc, hw[v / 2]);
      }
      const vec bhi = pairs_to_vec<NP>(hw), blo = pairs_to_vec<NP>(lw);
#pragma unroll
      for (int m = 0; m < F::MT; ++m) {
        acc[i][m] = mfma<NP>(ahi[m][ks], bhi, acc[i][m]);
        acc[i][m] = mfma<NP>(alo[m][ks], bhi, acc[i][m]);
        acc[i][m] = mfma<NP>(ahi[m][ks], blo, acc[i][m]);
      }
    }
#pragma unroll
    for (int m = 0; m < F::MT; ++m) acc[i][m] *= unscale;
  }
}

// The same with one power-of-two input scale `sc` for every column, chosen
// by the caller from a bound on the inputs (|x sc| < 2^15), and the output
// scale `post`.
template <int NP>
__device__ __forceinline__ void contract4_fixed(const typename Frag<NP>::vec (&ahi)[Frag<NP>::MT][Frag<NP>::KSTEPS],
                                                const typename Frag<NP>::vec (&alo)[Frag<NP>::MT][Frag<NP>::KSTEPS],
                                                float (&xv)[4][Frag<NP>::KSTEPS][Frag<NP>::KV],
                                                f32x4 (&acc)[4][Frag<NP>::MT], float sc, float post) {
  using F = Frag<NP>;
  using vec = typename F::vec;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 0; m < F::MT; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks) {
      uint32_t hw[F::KV / 2], lw[F::KV / 2];
#pragma unroll
      for (int v = 0; v < F::KV; v += 2) {
        hw[v / 2] = split_hi_pair(xv[i][ks][v], sc, xv[i][ks][v + 1], sc);
        lw[v / 2] = split_lo_pair(xv[i][ks][v], sc, xv[i][ks][v + 1], sc, hw[v / 2]);
      }
      const vec bhi = pairs_to_vec<NP>(hw), blo = pairs_to_vec<NP>(lw);
#pragma unroll
      for (int m = 0; m < F::MT; ++m) {
        acc[i][m] = mfma<NP>(ahi[m][ks], bhi, acc[i][m]);
        acc[i][m] = mfma<NP>(alo[m][ks], bhi, acc[i][m]);
        acc[i][m] = mfma<NP>(ahi[m][ks], blo, acc[i][m]);
      }
    }
#pragma unroll
    for (int m = 0; m < F::MT; ++m) acc[i][m] *= post;
  }
}

// Largest value over the wave
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// The Lloyd-Max levels are below 8 in magnitude (a bound the decode pass's
// fixed scaling relies on)
constexpr float kLevelsHost[] = {TACT_CODEBOOK_LEVEL_VALUES};
constexpr bool levels_below(float lim) {
  for (float v : kLevelsHost)
    if (v >= lim || v <= -lim) return false;
  return true;
}
static_assert(levels_below(8.0f), "decode scaling assumes |level| < 8");

// Persistent blocks of 8 waves (256 VGPRs each), each walking a list of
// planes.  While one plane is transformed, the data of the block's next
// plane is fetched into the registers the wave has just consumed (forward:
// the H columns of its w; inverse: the record words and side info of its kh
// rows), so memory and compute overlap.
constexpr int kPlaneWaves = 8;
// the decode pass runs 12 waves (3 per SIMD) on planes of 17..24 rows and
// columns: two rows and two columns per wave, 146 VGPRs
constexpr int kDecodeWaves = 12;

// The decoding walk is XCD-aware.  Workgroups are dispatched to the 8 XCDs
// round robin (block b runs on XCD b % 8) and every XCD has its own L2.  The
// 64-channel slabs of one slice read the same record lines (side info and
// code words of bins of consecutive heads are adjacent); spread over XCDs,
// every L2 would fetch them all.  So in decoding an XCD takes whole slices:
// XCD x walks slices x, x + 8, x + 16, ... slab by slab, and its blocks take
// the planes of that list in turn (the grid holds at least 8 blocks).  The
// forward walk shares no input lines between slabs and keeps the plain order
// (one group: block b takes planes b, b + grid, ...).
constexpr int kXcds = 8;

// Decode staging of one plane row: bin kw takes 5 16-byte slots ({bits,
// gain, first level-table entry, 0}, then its 64 code bytes, channel c at
// byte c), and 12 more slots follow every 8 bins, so that the four bins
// one W-stage read serves (kw, kw + 8, kw + 16, kw + 24) sit 52 slots
// (208 words, 16 banks mod 64) apart: their 16-lane code reads fall in
// distinct banks.
__host__ __device__ constexpr int decode_stage_slot(int kw) { return kw * 5 + (kw >> 3) * 12; }
// bytes of a row's staging for nk bins
__host__ __device__ constexpr int decode_stage_bytes(int nk) { return (decode_stage_slot(nk - 1) + 5) * 16; }

template <int GROUPS>
// Plane indices fit in 32 bits: a launch covers at most one workspace chunk
// of units (24 GiB of fp32 volume, under 2^28 planes of >= 64 entries), so
// the index arithmetic runs in 32-bit unsigned integers.
struct PlaneWalk {
  uint32_t n_slabs, n_slices, per_group;
  int group;
  // plane of position k in this block's group list, or -1 past its end
  __device__ __forceinline__ int64_t at(uint32_t k) const {
    const uint32_t slice = (k / n_slabs) * GROUPS + group;
    return slice < n_slices ? static_cast<int64_t>(slice * n_slabs + k % n_slabs) : -1;
  }
};

// plane p -> (unit, slice s, 64-channel slab): slab fastest
struct PlaneId {
  int64_t u;
  int s;
  int64_t c0;      // first channel of the slab
  int64_t head;
  int half;        // 64-channel word of the head
  int64_t vol;     // element offset of (u, s, 0, 0, 0)
};

__device__ __forceinline__ PlaneId plane_id(const PlaneArgs& a, int64_t p64) {
  const uint32_t p = static_cast<uint32_t>(p64);
  const uint32_t n_slabs = static_cast<uint32_t>(a.C / 64);
  PlaneId id;
  const uint32_t slab = p % n_slabs;
  const uint32_t rest = p / n_slabs;
  id.s = static_cast<int>(rest % static_cast<uint32_t>(a.S));
  id.u = rest / static_cast<uint32_t>(a.S);
  id.c0 = static_cast<int64_t>(slab) * 64;
  id.head = id.c0 / a.head_dim;
  id.half = static_cast<int>((id.c0 % a.head_dim) / 64);
  id.vol = id.u * a.ustride + static_cast<int64_t>(id.s) * a.H * a.W * a.C;
  return id;
}

template <int NPH, int NPW, int MODE, int SL, int WV>
__global__ __launch_bounds__(64 * WV) void k_plane(PlaneArgs a) {
  constexpr int kWaves = WV;
  using FH = Frag<NPH>;
  using FW = Frag<NPW>;
  // w columns (H passes) and kh rows (W passes) per wave: SL covers
  // ceil(max(H, W) / 8)
  constexpr int SLW = (SL < (NPW + kWaves - 1) / kWaves) ? SL : (NPW + kWaves - 1) / kWaves;
  constexpr int SLH = (SL < (NPH + kWaves - 1) / kWaves) ? SL : (NPH + kWaves - 1) / kWaves;
  // [H][W][64] fp32; 16-byte aligned so that float4 accesses are single
  // 128-bit LDS operations (a 16-lane group then covers all 64 banks once)
  extern __shared__ float4 plane_v4[];
  float* plane = reinterpret_cast<float*>(plane_v4);
  const int lane = threadIdx.x % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
  const int t = lane % 16, g = lane / 16;
  const int H = a.H, W = a.W;
  constexpr int kGroups = MODE == MODE_DEQUANT ? kXcds : 1;
  PlaneWalk<kGroups> walk;
  walk.n_slabs = static_cast<uint32_t>(a.C / 64);
  walk.n_slices = static_cast<uint32_t>(a.n_units * a.S);
  walk.group = static_cast<int>(blockIdx.x % kGroups);
  walk.per_group = (gridDim.x - walk.group + kGroups - 1) / kGroups;
  const uint32_t k0 = blockIdx.x / kGroups;
  // byte strides of a slice: one w step, one h row; this lane's columns
  const int cbytes = static_cast<int>(a.C) * 4;
  const int row_bytes = W * cbytes;
  // LDS row stride in 64-float positions: the decode pass stages NPW bins
  // in a row's area (decode_stage_bytes), so short rows are padded
  const int RW = MODE == MODE_DEQUANT ? max(W, (decode_stage_bytes(NPW) + 255) / 256) : W;
  // bin of (s, kh, kw) of a plane's head
  auto bin_of3 = [&](const PlaneId& id, int kh, int kw) -> int64_t {
    return ((static_cast<int64_t>(id.s) * H + kh) * W + kw) * a.kv_heads + id.head;
  };
  constexpr float kOne[4] = {1.f, 1.f, 1.f, 1.f};
  const int wpp = a.head_dim / 64;

  __shared__ FragLds<NPH> s_fh;
  // W axis: forward, split fragments (FragLds<NPW>); inverse, the fp32
  // matrix values per lane, [m][ks][v][lane], scaled per row by the bins'
  // gains, and the levels as (hi, lo) fp16 pairs with a zero entry first
  constexpr int kAwFloats = FW::MT * FW::KSTEPS * FW::KV * kWave;
  constexpr int kWBufWords = (MODE == MODE_DEQUANT)
                                 ? kAwFloats + TACT_CODEBOOK_LEVELS + 1
                                 : static_cast<int>(sizeof(FragLds<NPW>) / 4);
  __shared__ __attribute__((aligned(16))) uint32_t s_wbuf[kWBufWords];
  // where a stage writes its output rows or columns past H or W (dropped)
  __shared__ __attribute__((aligned(16))) float s_sink[4 * kWave];
  // statistics pass: a wave's row of partial sums (up to 32 bins), gathered
  // so that the row goes out in one store
  __shared__ float s_vsum[MODE == MODE_STATS ? kWaves * 32 : 1];
  FragLds<NPW>& s_fw = *reinterpret_cast<FragLds<NPW>*>(s_wbuf);
  float* s_aw = reinterpret_cast<float*>(s_wbuf);
  uint32_t* s_lp = s_wbuf + kAwFloats;
  if (wv == 0) {
    frag_to_lds<NPH>(s_fh, a.tab + 1 * 4096, MODE == MODE_DEQUANT, lane);
    if constexpr (MODE == MODE_DEQUANT) {
      const float* tw = a.tab + 2 * 4096;
#pragma unroll
      for (int m = 0; m < FW::MT; ++m)
#pragma unroll
        for (int ks = 0; ks < FW::KSTEPS; ++ks)
#pragma unroll
          for (int v = 0; v < FW::KV; ++v) {
            const int row = 16 * m + t;                       // output w
            const int col = ks * FW::KPER + FW::KV * g + v;   // input kw
            s_aw[((m * FW::KSTEPS + ks) * FW::KV + v) * kWave + lane] = kMatScale * tw[col * 64 + row];
          }
    } else {
      frag_to_lds<NPW>(s_fw, a.tab + 2 * 4096, 0, lane);
    }
  }
  if constexpr (MODE == MODE_DEQUANT) {
    for (int j = threadIdx.x; j <= TACT_CODEBOOK_LEVELS; j += blockDim.x) {
      uint32_t pr = 0;
      if (j > 0) {
        // scaled by 2^11 so that the low half of the smallest level (about
        // 0.01 at 8 bits) stays a normal fp16 number; |2^11 L| < 2^14
        const float lv = kLevelScale * c_levels[j - 1];
        _Float16 h, l;
        split2(lv, h, l);
        pr = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l)) << 16);
      }
      s_lp[j] = pr;
    }
  }
  __syncthreads();                           // fragments and tables in LDS

  if constexpr (MODE != MODE_DEQUANT) {
    // the H columns (all h, 64 channels) of this wave's w = wv + 8 j
    float xs[SLW][4][FH::KSTEPS][FH::KV];
    auto fetch_cols = [&](int64_t p, int j) {
      const PlaneId id = plane_id(a, p);
      const int w = wv + kWaves * j;
      // the slice as a buffer: rows h >= H read as 0
      const __amdgpu_buffer_rsrc_t rin = make_rsrc(a.in + id.vol, static_cast<int64_t>(row_bytes) * H);
      const int voff = (FH::KV * g * W + w) * cbytes + static_cast<int>(id.c0 + 4 * t) * 4;
#pragma unroll
      for (int ks = 0; ks < FH::KSTEPS; ++ks)
#pragma unroll
        for (int v = 0; v < FH::KV; ++v) {
          const float4 q = buf_ld4(rin, voff, (ks * FH::KPER + v) * row_bytes);
          xs[j][0][ks][v] = q.x; xs[j][1][ks][v] = q.y; xs[j][2][ks][v] = q.z; xs[j][3][ks][v] = q.w;
        }
    };
    int64_t p = walk.at(k0);
    if (p >= 0) {
#pragma unroll
      for (int j = 0; j < SLW; ++j)
        if (wv + kWaves * j < W) fetch_cols(p, j);
    }
    for (uint32_t k = k0; p >= 0; k += walk.per_group) {
      const PlaneId id = plane_id(a, p);
      const int64_t pn = walk.at(k + walk.per_group);
      const bool more = pn >= 0;
      const __amdgpu_buffer_rsrc_t rcoef =
          make_rsrc(a.out + id.vol, static_cast<int64_t>(row_bytes) * H);
      // ---- H axis: registers -> LDS; then fetch the next plane's columns
#pragma unroll
      for (int j = 0; j < SLW; ++j) {
        const int w = wv + kWaves * j;
        if (w >= W) break;
        f32x4 acc[4][FH::MT];
        typename FH::vec ahi[FH::MT][FH::KSTEPS], alo[FH::MT][FH::KSTEPS];
        frag_from_lds<NPH>(s_fh, lane, ahi, alo);
        contract4<NPH>(ahi, alo, xs[j], acc, kOne);
#pragma unroll
        for (int m = 0; m < FH::MT; ++m)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int kh = 16 * m + 4 * g + rr;
            lds_st4(kh < H ? plane + (kh * W + w) * 64 + 4 * t : s_sink + 4 * lane,
                    float4{acc[0][m][rr], acc[1][m][rr], acc[2][m][rr], acc[3][m][rr]});
          }
        if (more) fetch_cols(pn, j);
      }
      __syncthreads();
      // ---- W axis: LDS -> epilogue; a wave owns the columns of one kh ----
#pragma unroll
      for (int r = 0; r < SLH; ++r) {
        const int kh = wv + kWaves * r;
        if (kh >= H) break;
        float xv[4][FW::KSTEPS][FW::KV];
#pragma unroll
        for (int ks = 0; ks < FW::KSTEPS; ++ks)
#pragma unroll
          for (int v = 0; v < FW::KV; ++v) {
            // K rows w >= W read row W - 1: the zero-padded matrix column
            // takes them out of the product (no predicate)
            const int w = ks * FW::KPER + FW::KV * g + v;
            const float4 q = lds_ld4(plane + (kh * W + (w < W ? w : W - 1)) * 64 + 4 * t);
            xv[0][ks][v] = q.x; xv[1][ks][v] = q.y; xv[2][ks][v] = q.z; xv[3][ks][v] = q.w;
          }
        f32x4 acc[4][FW::MT];
        typename FW::vec bhi_w[FW::MT][FW::KSTEPS], blo_w[FW::MT][FW::KSTEPS];
        frag_from_lds<NPW>(s_fw, lane, bhi_w, blo_w);
        contract4<NPW>(bhi_w, blo_w, xv, acc, kOne);
        {
          // partial sums of bin (s, kh, kw, head), plane by plane: a row's
          // sums are adjacent
          float* vrow = a.var_part + id.u * a.var_stride +
                        ((id.c0 / 64 * a.S + id.s) * static_cast<int64_t>(H) + kh) * W;
          // the final coefficients go back over this plane's input
          const int vo = (kh * W + 4 * g) * cbytes + static_cast<int>(id.c0 + 4 * t) * 4;
#pragma unroll
          for (int m = 0; m < FW::MT; ++m)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              float sq = 0.f;
#pragma unroll
              for (int i = 0; i < 4; ++i) sq = fmaf(acc[i][m][rr], acc[i][m][rr], sq);
              sq = row_sum16(sq);
              const int kw = 16 * m + 4 * g + rr;
              if (t == 0) s_vsum[wv * 32 + kw] = sq;
              // columns past W take an offset past the buffer (dropped)
              buf_st4<2>(rcoef, kw < W ? vo : kPastBuffer, (16 * m + rr) * cbytes,
                         float4{acc[0][m][rr], acc[1][m][rr], acc[2][m][rr], acc[3][m][rr]});
            }
          // the row's sums, lane kw (one store instead of one per sum)
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          if (lane < W) vrow[lane] = s_vsum[wv * 32 + lane];
        }
      }
      __syncthreads();                       // LDS free for the next plane
      p = pn;
    }
  } else {
    // Side info (bits, first plane, gain) and code words of this wave's kh
    // rows, fetched one plane ahead: lane (r, kw), r = lane / 32, holds bin
    // (kh, kw) of the wave's row q = 2 ps + r in pass ps (two rows at once,
    // so that a plane row of up to 32 bins keeps half the wave busy).
    constexpr int kPass = (SLH + 1) / 2;
    const int srow = lane / 32, skw = lane % 32;
    int bj[kPass], pjv[kPass];
    float gjv[kPass];
    uint2 wd[kPass][8];
    // Record reads through buffer descriptors (32-bit offsets per lane).
    // Every call issues the same loads: lanes with nothing to read take an
    // offset past the buffer and read 0.  With fixed load and store counts
    // the compiler's waits count the stores issued after a load instead of
    // waiting for all memory operations.
    auto fetch_side = [&](int64_t p) {
      const PlaneId id = plane_id(a, p);
      const uint8_t* r = a.rec.base + id.u * a.rec.stride;
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(r + a.rec.off_bits, a.n_bins);
      const __amdgpu_buffer_rsrc_t rg = make_rsrc(r + a.rec.off_gains, 4 * a.n_bins);
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.plane_off + id.u * a.n_bins, 4 * a.n_bins);
#pragma unroll
      for (int ps = 0; ps < kPass; ++ps) {
        const int q = 2 * ps + srow;
        const int kh = wv + kWaves * q;
        const bool ok = q < SLH && kh < H && skw < W;
        const int bin = static_cast<int>(bin_of3(id, ok ? kh : 0, ok ? skw : 0));
        const int vb = ok ? bin : kPastBuffer, vw = ok ? 4 * bin : kPastBuffer;
        bj[ps] = __builtin_amdgcn_raw_buffer_load_b8(rb, vb, 0, 0);
        pjv[ps] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(ro, vw, 0, 0));
        gjv[ps] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, vw, 0, 0));
      }
    };
    auto fetch_words = [&](int64_t p) {
      const PlaneId id = plane_id(a, p);
      // the plane words of this slab: 64-bit word (plane * wpp + half)
      const __amdgpu_buffer_rsrc_t rw =
          make_rsrc(a.rec.base + id.u * a.rec.stride + a.rec.off_codes, a.total_bits * wpp * 8);
#pragma unroll
      for (int ps = 0; ps < kPass; ++ps) {
        int b = bj[ps];
        const int64_t pj = static_cast<uint32_t>(pjv[ps]);
        if (b > a.max_bits || pj + b > a.total_bits) b = 0;
        bj[ps] = b;
        const int base = 8 * (static_cast<int>(pj) * wpp + id.half);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          wd[ps][k] = __builtin_bit_cast(
              uint2, __builtin_amdgcn_raw_buffer_load_b64(rw, k < b ? base + 8 * wpp * k : kPastBuffer, 0, 0));
      }
    };
    // Largest gain of a coded bin of the plane, per wave, for the scaling of
    // both stages; written one plane ahead, slot = plane count parity
    __shared__ float s_gmax[2][kWaves];
    auto gain_max = [&]() {
      float m = 0.f;
#pragma unroll
      for (int ps = 0; ps < kPass; ++ps) m = fmaxf(m, bj[ps] > 0 ? gjv[ps] : 0.f);
      return wave_max(m);
    };
    int64_t p = walk.at(k0);
    if (p >= 0) {
      fetch_side(p);
      fetch_words(p);
      const float m = gain_max();
      if (lane == 0) s_gmax[0][wv] = m;
      // As many stores as the H stage issues, through an empty buffer (all
      // dropped): the loop is entered with the same number of memory
      // operations after the code-word loads as its back edge carries, so
      // the compiler's wait for those loads at the loop top counts the
      // stores instead of waiting for them.
      const __amdgpu_buffer_rsrc_t none = make_rsrc(a.out, 0);
#pragma unroll
      for (int j = 0; j < SLW * FH::MT * 4; ++j) buf_st4(none, 0, 0, float4{0.f, 0.f, 0.f, 0.f});
    }
    __syncthreads();
    for (uint32_t k = k0, it = 0; p >= 0; k += walk.per_group, ++it) {
      const PlaneId id = plane_id(a, p);
      const int64_t pn = walk.at(k + walk.per_group);
      const bool more = pn >= 0;
      // Plane scaling from gmax, the largest gain of a coded bin, with
      // gmax < 2^e (e >= -100): A' = (2^12 C^T) diag(g) 2^(2 - e), so
      // |A'| < 2^14, and the levels scaled by 2^11 (|2^11 L| < 2^14) give
      // W-stage outputs 2^(25 - e) x.  As |L| < 8 and a row of C^T has at
      // most 32 entries of unit norm (sum of |c| < 2^3), |x| < 2^(e + 6):
      // the outputs stay below 2^31 and enter the H stage scaled by 2^-17.
      // The H-stage outputs are then 2^12 2^-17 2^(25 - e) y = 2^(20 - e) y.
      float gmax = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < kWaves; ++w8) gmax = fmaxf(gmax, s_gmax[it & 1][w8]);
      int e = 0;
      if (gmax > 0.f) frexpf(gmax, &e);
      e = e < -100 ? -100 : e;
      const float gsc = ldexpf(1.0f, 2 - e);
      const float yscale = ldexpf(1.0f, e - 20);
      // ---- inverse W: decode into the B fragments, contract; a wave owns one
      // kh row.  The row's LDS area first holds its bins' staging, 80 bytes
      // per bin (decode_stage_slot): {bits, gain, first level-table entry,
      // 0}, then the bin's 64 codes, one byte per channel (planes at or above
      // the bin's bit width are 0; bins without bits have gain 0).  The
      // staging lane of a bin turns its bit planes into code bytes (two
      // 32-channel plane transpositions, for as many planes as the wave's
      // widest bin has), and lane (t, g) of the W stage reads the 4 code
      // bytes of its channels 4t..4t+3 for each of its K rows kw.
      //   All rows are staged first.  The next plane's side info is then
      // fetched, and its code words at the end of this W stage: both before
      // this plane's stores.  Vector memory operations complete in issue
      // order, so waiting for those loads never waits for the stores, which
      // drain during the next W stage.
      {
        // planes to transpose: the widest bin of the wave, rounded up to 1,
        // 2, 4 or 8 (narrower bins have zero planes there)
        int bw = 0;
#pragma unroll
        for (int ps = 0; ps < kPass; ++ps) bw = max(bw, bj[ps]);
        const bool nb8 = __ballot(bw > 4) != 0;
        const bool nb4 = __ballot(bw > 2) != 0;
        const bool nb2 = __ballot(bw > 1) != 0;
#pragma unroll
        for (int ps = 0; ps < kPass; ++ps) {
          uint32_t pl[8], ph[8], ql[8], qh[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            pl[k] = wd[ps][k].x;
            ph[k] = wd[ps][k].y;
          }
          if (nb8) {
            planes_to_codes<8>(pl, ql);
            planes_to_codes<8>(ph, qh);
          } else if (nb4) {
            planes_to_codes<4>(pl, ql);
            planes_to_codes<4>(ph, qh);
          } else if (nb2) {
            planes_to_codes<2>(pl, ql);
            planes_to_codes<2>(ph, qh);
          } else {
            planes_to_codes<1>(pl, ql);
            planes_to_codes<1>(ph, qh);
          }
          const int q = 2 * ps + srow;
          const int kh = wv + kWaves * q;
          // K rows W..NPW-1 are staged as empty bins (nothing was read)
          if (q < SLH && kh < H && skw < NPW) {
            uint4* st = reinterpret_cast<uint4*>(plane + static_cast<int64_t>(kh) * RW * 64);
            const int b = bj[ps];
            const int sl = decode_stage_slot(skw);
            st[sl] = uint4{static_cast<uint32_t>(b), b > 0 ? __float_as_uint(gjv[ps]) : 0u,
                           b > 0 ? (1u << b) - 1u : 0u, 0u};
            st[sl + 1] = uint4{ql[0], ql[1], ql[2], ql[3]};
            st[sl + 2] = uint4{ql[4], ql[5], ql[6], ql[7]};
            st[sl + 3] = uint4{qh[0], qh[1], qh[2], qh[3]};
            st[sl + 4] = uint4{qh[4], qh[5], qh[6], qh[7]};
          }
        }
      }
      // (the last plane of the walk fetches itself again: same loads, unused)
      const int64_t pf = more ? pn : p;
      fetch_side(pf);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int q = 0; q < SLH; ++q) {
        const int kh = wv + kWaves * q;
        if (kh >= H) break;
        float* row = plane + static_cast<int64_t>(kh) * RW * 64;
        const uint4* st = reinterpret_cast<const uint4*>(row);
        // B = the levels as (hi, lo) fp16 pairs; the gains go into A
        uint32_t bp[4][FW::KSTEPS][FW::KV];
        float gv[FW::KSTEPS][FW::KV];
#pragma unroll
        for (int ks = 0; ks < FW::KSTEPS; ++ks)
#pragma unroll
          for (int v = 0; v < FW::KV; ++v) {
            // (K rows kw >= W are staged as empty bins)
            const int kw = ks * FW::KPER + FW::KV * g + v;
            const int sl = decode_stage_slot(kw);
            const uint4 sb = st[sl];
            // byte i: the code of channel 4t + i
            const uint32_t codes = reinterpret_cast<const uint32_t*>(st + sl + 1)[t];
            gv[ks][v] = __uint_as_float(sb.y);
            const int base = static_cast<int>(sb.z);           // s_lp[0] = 0
#pragma unroll
            for (int i = 0; i < 4; ++i) bp[i][ks][v] = s_lp[base + static_cast<int>((codes >> (8 * i)) & 0xFFu)];
          }
        // every lane has read the staging before the outputs overwrite it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // A' split into fp16 hi / lo
        typename FW::vec ahi_w[FW::MT][FW::KSTEPS], alo_w[FW::MT][FW::KSTEPS];
        const int la = opaque(lane);
#pragma unroll
        for (int ks = 0; ks < FW::KSTEPS; ++ks)
#pragma unroll
          for (int v = 0; v < FW::KV; ++v) gv[ks][v] *= gsc;
#pragma unroll
        for (int m = 0; m < FW::MT; ++m)
#pragma unroll
          for (int ks = 0; ks < FW::KSTEPS; ++ks) {
            uint32_t hw[FW::KV / 2], lw[FW::KV / 2];
#pragma unroll
            for (int v = 0; v < FW::KV; v += 2) {
              const float* c = s_aw + ((m * FW::KSTEPS + ks) * FW::KV + v) * kWave + la;
              hw[v / 2] = split_hi_pair(c[0], gv[ks][v], c[kWave], gv[ks][v + 1]);
              lw[v / 2] = split_lo_pair(c[0], gv[ks][v], c[kWave], gv[ks][v + 1], hw[v / 2]);
            }
            ahi_w[m][ks] = pairs_to_vec<NPW>(hw);
            alo_w[m][ks] = pairs_to_vec<NPW>(lw);
          }
        f32x4 acc[4][FW::MT];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int m = 0; m < FW::MT; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < FW::KSTEPS; ++ks) {
            typename FW::vec bhi, blo;
#pragma unroll
            for (int v = 0; v < FW::KV; ++v) {
              bhi[v] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bp[i][ks][v] & 0xFFFFu));
              blo[v] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bp[i][ks][v] >> 16));
            }
#pragma unroll
            for (int m = 0; m < FW::MT; ++m) {
              acc[i][m] = mfma<NPW>(ahi_w[m][ks], bhi, acc[i][m]);
              acc[i][m] = mfma<NPW>(alo_w[m][ks], bhi, acc[i][m]);
              acc[i][m] = mfma<NPW>(ahi_w[m][ks], blo, acc[i][m]);
            }
          }
        }
        // output columns w >= W go to a per-lane sink (no predicate)
#pragma unroll
        for (int m = 0; m < FW::MT; ++m)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int w = 16 * m + 4 * g + rr;
            lds_st4(w < W ? row + w * 64 + 4 * t : s_sink + 4 * lane,
                    float4{acc[0][m][rr], acc[1][m][rr], acc[2][m][rr], acc[3][m][rr]});
          }
      }
      fetch_words(pf);
      {
        const float m = gain_max();          // of the next plane
        if (lane == 0) s_gmax[(it + 1) & 1][wv] = m;
      }
      __syncthreads();
      // ---- inverse H: LDS -> global; a wave owns the columns of one w -----
      // Every wave issues the same stores: a column past W is computed from
      // column W - 1 and stored through an empty buffer (dropped).
#pragma unroll
      for (int j = 0; j < SLW; ++j) {
        const bool wok = wv + kWaves * j < W;
        const int w = wok ? wv + kWaves * j : W - 1;
        const __amdgpu_buffer_rsrc_t rout =
            make_rsrc(a.out + id.vol, wok ? static_cast<int64_t>(row_bytes) * H : 0);
        float xv[4][FH::KSTEPS][FH::KV];
#pragma unroll
        for (int ks = 0; ks < FH::KSTEPS; ++ks)
#pragma unroll
          for (int v = 0; v < FH::KV; ++v) {
            // K rows kh >= H read row H - 1: the zero-padded matrix column
            // takes them out of the product (no predicate)
            const int kh = ks * FH::KPER + FH::KV * g + v;
            const float4 qv = lds_ld4(plane + ((kh < H ? kh : H - 1) * RW + w) * 64 + 4 * t);
            xv[0][ks][v] = qv.x; xv[1][ks][v] = qv.y; xv[2][ks][v] = qv.z; xv[3][ks][v] = qv.w;
          }
        f32x4 acc[4][FH::MT];
        typename FH::vec ahi_h[FH::MT][FH::KSTEPS], alo_h[FH::MT][FH::KSTEPS];
        frag_from_lds<NPH>(s_fh, lane, ahi_h, alo_h);
        contract4_fixed<NPH>(ahi_h, alo_h, xv, acc, 0x1p-17f, yscale);
        // rows h >= H fall past the buffer's range and are dropped
        const int voff = (4 * g * W + w) * cbytes + static_cast<int>(id.c0 + 4 * t) * 4;
#pragma unroll
        for (int m = 0; m < FH::MT; ++m)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            buf_st4<2>(rout, voff, (16 * m + rr) * row_bytes,
                    float4{acc[0][m][rr], acc[1][m][rr], acc[2][m][rr], acc[3][m][rr]});
      }
      __syncthreads();                       // LDS free for the next plane
      p = pn;
    }
  }
}

// ---------------------------------------------------------------------------
// Allocation by exact radix selection.
// Gains of bin i are key_i - (k-1) * 2^53 (k = 1..bmax) in the bit pattern of
// the fp64 value var_i * 4^-(k-1); key_i = pattern of (double)var_i, or 0 for
// var_i == 0.  As (exponent e, mantissa) pairs a gain is (E_i - 2(k-1), M_i).
// Sweep 1 finds the exponent of the T-th largest gain from a histogram of
// E_i, sweeps 2-3 find its mantissa (only the top 23 mantissa bits can be
// non-zero: the values come from fp32), then the final sweep assigns bits,
// breaking ties at the cut by bin index, and writes the record header and
// per-bin plane offsets.
// ---------------------------------------------------------------------------
constexpr int kAllocThreads = 512;

__device__ __forceinline__ uint64_t gain_key(float v) {
  return v > 0.f ? static_cast<uint64_t>(__double_as_longlong(static_cast<double>(v))) : 0ull;
}

__device__ __forceinline__ int count_ge(uint64_t key, uint64_t tau, int bmax) {
  if (key == 0) return tau == 0 ? bmax : 0;
  if (key < tau) return 0;
  const uint64_t q = ((key - tau) >> 53) + 1;
  return q > static_cast<uint64_t>(bmax) ? bmax : static_cast<int>(q);
}

// exclusive scan over the block (thread order), returns total via *total
__device__ int block_exscan(int v, int* sh, int* total) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  __syncthreads();
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < static_cast<int>(blockDim.x) / kWave; ++i) {
    if (i < w) before += sh[i];
    all += sh[i];
  }
  *total = all;
  return before + incl - v;
}

// Largest bucket b of hist[0..nb) with sum_{y >= b} hist[y] >= need; the
// count strictly above it goes to *above.  nb <= 4 * blockDim.x.
__device__ void select_bucket(const uint32_t* hist, int nb, int64_t need, int* sh,
                              int* out_bucket, int64_t* out_above) {
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int hi = nb - 1 - static_cast<int>(threadIdx.x) * per;
  int mine = 0;
  for (int j = 0; j < per; ++j)
    if (hi - j >= 0) mine += hist[hi - j];
  int tot;
  const int before = block_exscan(mine, sh, &tot);
  __shared__ int s_bucket;
  __shared__ long long s_above;
  if (threadIdx.x == 0) {
    s_bucket = -1;
    s_above = 0;
  }
  __syncthreads();
  int64_t run = before;
  for (int j = 0; j < per; ++j) {
    const int b = hi - j;
    if (b < 0) break;
    const int64_t after = run + hist[b];
    if (run < need && after >= need) {
      s_bucket = b;
      s_above = run;
    }
    run = after;
  }
  __syncthreads();
  *out_bucket = s_bucket;
  *out_above = s_above;
  __syncthreads();
}

// The variance of bins i0..i0+3: (sum of the `parts` partial sums, added in
// part order) * scale.  Partials of a bin are consecutive.
__device__ __forceinline__ void var4(const float* v, int64_t nb, int parts, float scale,
                                     bool vec, int64_t i0, float (&out)[4]) {
  if (vec && i0 + 3 < nb) {
    if (parts == 1) {
      const float4 q = *reinterpret_cast<const float4*>(v + i0);
      out[0] = q.x; out[1] = q.y; out[2] = q.z; out[3] = q.w;
    } else if (parts == 2) {
      const float4 q0 = *reinterpret_cast<const float4*>(v + 2 * i0);
      const float4 q1 = *reinterpret_cast<const float4*>(v + 2 * i0 + 4);
      out[0] = q0.x + q0.y; out[1] = q0.z + q0.w; out[2] = q1.x + q1.y; out[3] = q1.z + q1.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 q = *reinterpret_cast<const float4*>(v + 4 * (i0 + j));
        out[j] = ((q.x + q.y) + q.z) + q.w;
      }
    }
  } else {
    for (int j = 0; j < 4; ++j) {
      float acc = 0.f;
      if (i0 + j < nb) {
        acc = v[(i0 + j) * parts];
        for (int p = 1; p < parts; ++p) acc += v[(i0 + j) * parts + p];
      }
      out[j] = acc;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] *= scale;
}

// Partial sums stored plane by plane: [slab][position], slab = head * parts
// + part, position = bin / kv_heads (the bin is position * kv_heads + head).
// The variance adds the parts in part order, as var4 does.
struct VarView {
  const float* v;
  int64_t nb, npos;
  int parts, kv;
  bool planes, vec;
  __device__ __forceinline__ float at(int h, int64_t pos, float scale) const {
    const float* q = v + static_cast<int64_t>(h) * parts * npos + pos;
    float acc = q[0];
    for (int p = 1; p < parts; ++p) acc += q[p * npos];
    return acc * scale;
  }
};

// Calls f(v_i) for the bins of one slice of a unit, in no particular order:
// 4 consecutive entries per thread per step, in the order of the storage.
// The slice is [lo, hi) in storage units: bins, or (plane by plane)
// positions of every head; lo is a multiple of 4, hi too unless it is the end.
template <typename Fn>
__device__ __forceinline__ void for_bins4(const VarView& vv, float scale, int64_t lo, int64_t hi,
                                          Fn f) {
  if (!vv.planes) {
    for (int64_t i0 = lo + 4 * static_cast<int64_t>(threadIdx.x); i0 < hi; i0 += 4 * blockDim.x) {
      float q[4];
      var4(vv.v, vv.nb, vv.parts, scale, vv.vec, i0, q);
      for (int j = 0; j < 4; ++j)
        if (i0 + j < hi) f(q[j]);
    }
    return;
  }
  // head by head, positions in storage order
  if (vv.vec && (vv.npos & 3) == 0) {
    // four groups of 4 positions per thread per step, all loads first (the
    // sweep is otherwise one load latency per group); indices past the slice
    // are clamped and their values unused
    const int64_t n4 = vv.npos / 4, g_lo = lo / 4, g_hi = hi / 4;
    if (g_hi <= g_lo) return;
    for (int h = 0; h < vv.kv; ++h) {
      const float4* q = reinterpret_cast<const float4*>(vv.v + static_cast<int64_t>(h) * vv.parts * vv.npos);
      for (int64_t g0 = g_lo + threadIdx.x; g0 < g_hi; g0 += 4 * static_cast<int64_t>(blockDim.x)) {
        float4 x0[4], x1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int64_t g = g0 + u * static_cast<int64_t>(blockDim.x);
          g = g < g_hi ? g : g_hi - 1;
          x0[u] = q[g];
          x1[u] = vv.parts > 1 ? q[n4 + g] : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t g = g0 + u * static_cast<int64_t>(blockDim.x);
          if (g >= g_hi) break;
          float4 acc = x0[u];
          if (vv.parts > 1) {
            acc.x += x1[u].x; acc.y += x1[u].y; acc.z += x1[u].z; acc.w += x1[u].w;
          }
          for (int p = 2; p < vv.parts; ++p) {
            const float4 r = q[p * n4 + g];
            acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
          }
          f(acc.x * scale); f(acc.y * scale); f(acc.z * scale); f(acc.w * scale);
        }
      }
    }
  } else {
    for (int h = 0; h < vv.kv; ++h)
      for (int64_t pos = lo + threadIdx.x; pos < hi; pos += blockDim.x) f(vv.at(h, pos, scale));
  }
}

// gains of exponent e for a bin with var exponent E (> 0): E = e + 2(k-1)
__device__ __forceinline__ bool has_gain_at(int E, int e, int bmax) {
  const int d = E - e;
  return E > 0 && d >= 0 && (d & 1) == 0 && d / 2 < bmax;
}

// Several workgroups per unit, each on a slice of its bins.  A unit's
// scratch holds the three sweeps' histograms, summed over the slices with
// integer atomics (so the sums do not depend on the order), the cut and the
// slices' totals; every kernel re-derives the cut from the histograms it
// needs, so all slices agree on it.
struct AllocArgs {
  Geometry g;
  const float* var;            // partial sums of squares, unit stride var_stride
  int64_t var_stride;
  int parts;                   // partial sums per bin
  float var_scale;
  int planes;                  // partials stored plane by plane (else per bin)
  uint8_t* scratch;            // kAllocScratchBytes per unit
  int64_t slice;               // bins per workgroup (a multiple of kAllocChunk and of 4 kv_heads)
  uint8_t* bits_out;
  RecordView rec;
  uint32_t* plane_off;
  float* inv_gain;
  float* var_out;
};
constexpr int kAllocChunk = 4 * kAllocThreads;      // bins per step of the final pass
// scratch layout (bytes): sweep histograms at 0 (2048 + 4096 + 2048 words),
// the cut at kAllocCutOff, the slice totals at kAllocTotOff
constexpr int64_t kAllocCutOff = 4 * 8192;
constexpr int64_t kAllocTotOff = kAllocCutOff + 256;
static_assert(kAllocTotOff + 16 * kAllocMaxSlices <= kAllocScratchBytes, "allocation scratch");

struct AllocCut {
  unsigned long long tau;      // the T-th largest gain's key
  long long need;              // gains equal to tau that get their bit
  long long eq_total;          // gains equal to tau
  int all_ties;                // need == eq_total
};

__device__ __forceinline__ VarView alloc_view(const AllocArgs& a, int64_t u) {
  VarView vv;
  vv.v = a.var + u * a.var_stride;
  vv.nb = a.g.n_bins;
  vv.npos = static_cast<int64_t>(a.g.S) * a.g.H * a.g.W;
  vv.parts = a.parts;
  vv.kv = a.g.kv_heads;
  vv.planes = a.planes != 0;
  vv.vec = (reinterpret_cast<uintptr_t>(vv.v) & 15) == 0;
  return vv;
}

// the storage slice [lo, hi) of workgroup w: bins, or positions of every head
__device__ __forceinline__ void alloc_storage_slice(const AllocArgs& a, const VarView& vv, int64_t w,
                                                    int64_t* lo, int64_t* hi) {
  if (vv.planes) {
    const int64_t per = a.slice / vv.kv;
    *lo = w * per;
    *hi = *lo + per < vv.npos ? *lo + per : vv.npos;
  } else {
    *lo = w * a.slice;
    *hi = *lo + a.slice < vv.nb ? *lo + a.slice : vv.nb;
  }
}

// The cut from the histograms of sweeps 1..stages (hist: 4096 words of LDS).
// Returns the stage reached: 1 with *ebin == 0 when the T-th largest gain is
// 0 (the cut is then complete), else the stages asked for.
__device__ __forceinline__ void alloc_cut(const uint32_t* G, int stages, int bmax, int64_t T, uint32_t* hist,
                          int* sh, int* ebin, int64_t* above, int* b2, int64_t* above2,
                          AllocCut* cut) {
  for (int j = threadIdx.x; j < 2048; j += blockDim.x) hist[j] = G[j];
  __syncthreads();
  // gains per exponent e: bins with E in {e, e+2, ..., e+2(bmax-1)} (E > 0);
  // all bmax gains of zero bins sit at e = 0
  for (int e = threadIdx.x; e < 2048; e += blockDim.x) {
    uint32_t c = 0;
    if (e == 0) {
      c = hist[0] * static_cast<uint32_t>(bmax);
    } else {
      for (int k = 0; k < bmax; ++k) {
        const int E = e + 2 * k;
        if (E < 2048) c += hist[E];
      }
    }
    hist[2048 + e] = c;
  }
  __syncthreads();
  select_bucket(hist + 2048, 2048, T, sh, ebin, above);
  if (*ebin == 0) {
    if (cut) {
      cut->tau = 0;
      cut->eq_total = hist[2048];
      cut->need = T - *above;
    }
    return;
  }
  if (stages < 2) return;
  // The keys hold the fp32 gains exactly in their top 35 bits, so tau, the
  // T-th largest gain, is fixed by the three digits, and the counts of the
  // gains above it and equal to it follow from the histograms.
  for (int j = threadIdx.x; j < 4096; j += blockDim.x) hist[j] = G[2048 + j];
  __syncthreads();
  select_bucket(hist, 4096, T - *above, sh, b2, above2);
  if (stages < 3) return;
  for (int j = threadIdx.x; j < 2048; j += blockDim.x) hist[j] = G[6144 + j];
  __syncthreads();
  int b3;
  int64_t above3;
  select_bucket(hist, 2048, T - *above - *above2, sh, &b3, &above3);
  cut->tau = (static_cast<uint64_t>(*ebin) << 52) | (static_cast<uint64_t>(*b2) << 40) |
             (static_cast<uint64_t>(b3) << 29);
  cut->need = T - (*above + *above2 + above3);
  cut->eq_total = hist[b3];
}

__global__ __launch_bounds__(256) void k_alloc_clear(uint8_t* scratch) {
  uint32_t* G = reinterpret_cast<uint32_t*>(scratch + blockIdx.x * kAllocScratchBytes);
  for (int j = threadIdx.x; j < 8192; j += blockDim.x) G[j] = 0;
}

// Sweep STAGE over one slice: the histogram of the gains' exponents (1), of
// the next 12 bits among gains at the cut's exponent (2), of the next 11 bits
// among those with the cut's 12 bits (3), added into the unit's histogram.
template <int STAGE>
__global__ __launch_bounds__(kAllocThreads) void k_alloc_hist(AllocArgs a) {
  __shared__ uint32_t hist[4096];
  __shared__ int sh[kAllocThreads / kWave];
  const int64_t u = blockIdx.y;
  uint32_t* G = reinterpret_cast<uint32_t*>(a.scratch + u * kAllocScratchBytes);
  const int bmax = a.g.max_bits;
  int ebin = 0, b2 = 0;
  int64_t above = 0, above2 = 0;
  if constexpr (STAGE >= 2) {
    alloc_cut(G, STAGE - 1, bmax, a.g.total_bits, hist, sh, &ebin, &above, &b2, &above2, nullptr);
    if (ebin == 0) return;                   // the cut is complete
    __syncthreads();
  }
  constexpr int NH = STAGE == 2 ? 4096 : 2048;
  for (int j = threadIdx.x; j < NH; j += blockDim.x) hist[j] = 0;
  __syncthreads();
  const VarView vv = alloc_view(a, u);
  int64_t lo, hi;
  alloc_storage_slice(a, vv, blockIdx.x, &lo, &hi);
  for_bins4(vv, a.var_scale, lo, hi, [&](float x) {
    const uint64_t key = gain_key(x);
    if constexpr (STAGE == 1) {
      atomicAdd(&hist[key >> 52], 1u);
    } else if constexpr (STAGE == 2) {
      if (has_gain_at(static_cast<int>(key >> 52), ebin, bmax)) atomicAdd(&hist[(key >> 40) & 0xFFF], 1u);
    } else {
      if (has_gain_at(static_cast<int>(key >> 52), ebin, bmax) &&
          static_cast<int>((key >> 40) & 0xFFF) == b2)
        atomicAdd(&hist[(key >> 29) & 0x7FF], 1u);
    }
  });
  __syncthreads();
  uint32_t* Gs = G + (STAGE == 1 ? 0 : STAGE == 2 ? 2048 : 6144);
  for (int j = threadIdx.x; j < NH; j += blockDim.x)
    if (hist[j]) atomicAdd(&Gs[j], hist[j]);
}

// Per slice: its bins' bits below the cut (count_ge(key, tau + 1)) and its
// gains equal to the cut; workgroup 0 of a unit also stores the cut.
__global__ __launch_bounds__(kAllocThreads) void k_alloc_count(AllocArgs a) {
  __shared__ uint32_t hist[4096];
  __shared__ int sh[kAllocThreads / kWave];
  __shared__ long long red[2][kAllocThreads / kWave];
  const int64_t u = blockIdx.y;
  uint8_t* sc = a.scratch + u * kAllocScratchBytes;
  const Geometry& g = a.g;
  const int bmax = g.max_bits;
  const bool wf = g.alloc_mode == TACT_ALLOC_WATERFILL && g.total_bits > 0;
  AllocCut cut{0ull, 0, 0, 1};
  if (wf) {
    int ebin, b2 = 0;
    int64_t above, above2 = 0;
    alloc_cut(reinterpret_cast<const uint32_t*>(sc), 3, bmax, g.total_bits, hist, sh, &ebin, &above,
              &b2, &above2, &cut);
    cut.all_ties = cut.need == cut.eq_total;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<AllocCut*>(sc + kAllocCutOff) = cut;
  const VarView vv = alloc_view(a, u);
  int64_t lo, hi;
  alloc_storage_slice(a, vv, blockIdx.x, &lo, &hi);
  long long nbits = 0, neq = 0;
  if (wf) {
    const uint64_t tau = cut.tau;
    for_bins4(vv, a.var_scale, lo, hi, [&](float x) {
      const uint64_t key = gain_key(x);
      const int b = count_ge(key, tau + 1, bmax);
      nbits += b;
      neq += count_ge(key, tau, bmax) - b;
    });
  } else if (g.alloc_mode == TACT_ALLOC_UNIFORM) {
    const int64_t bins = vv.planes ? (hi - lo) * vv.kv : hi - lo;
    if (threadIdx.x == 0) nbits = (hi > lo ? bins : 0) * static_cast<long long>(g.budget_bits);
  }
  // the slice's sums over the block
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    nbits += __shfl_xor(nbits, o, kWave);
    neq += __shfl_xor(neq, o, kWave);
  }
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  if (lane == 0) {
    red[0][wv] = nbits;
    red[1][wv] = neq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long tb = 0, te = 0;
    for (int j = 0; j < kAllocThreads / kWave; ++j) {
      tb += red[0][j];
      te += red[1][j];
    }
    long long* tot = reinterpret_cast<long long*>(sc + kAllocTotOff) + 2 * blockIdx.x;
    tot[0] = tb;
    tot[1] = te;
  }
}

// The final pass over one slice, in bin order: bits (ties at the cut by bin
// index, continuing the count of the slices before), record header, first
// planes, reciprocal gains and the variances; workgroup 0 also clears the
// record's padding.
__global__ __launch_bounds__(kAllocThreads) void k_alloc_write(AllocArgs a) {
  __shared__ float s_var[4 * kAllocThreads];   // one chunk of variances, bin order
  __shared__ int sh[kAllocThreads / kWave];
  const int64_t u = blockIdx.y;
  const uint8_t* sc = a.scratch + u * kAllocScratchBytes;
  const Geometry& g = a.g;
  const VarView vv = alloc_view(a, u);
  const int bmax = g.max_bits;
  const int64_t nb = g.n_bins;
  const bool wf = g.alloc_mode == TACT_ALLOC_WATERFILL && g.total_bits > 0;
  const AllocCut cut = *reinterpret_cast<const AllocCut*>(sc + kAllocCutOff);
  const uint64_t tau = cut.tau;
  const int64_t need = cut.need;
  const bool all_ties = cut.all_ties != 0;
  // ties and planes of the slices before this one
  const long long* tot = reinterpret_cast<const long long*>(sc + kAllocTotOff);
  int64_t tie_carry = 0, plane_carry = 0;
  for (int w = 0; w < static_cast<int>(blockIdx.x); ++w) {
    const long long nbits = tot[2 * w], neq = tot[2 * w + 1];
    long long take = neq;
    if (!all_ties) {
      take = need - tie_carry;
      take = take < 0 ? 0 : (take > neq ? neq : take);
    }
    tie_carry += neq;
    plane_carry += nbits + take;
  }
  const int64_t lo = static_cast<int64_t>(blockIdx.x) * a.slice;
  const int64_t hi = lo + a.slice < nb ? lo + a.slice : nb;
  uint8_t* bo = a.bits_out ? a.bits_out + u * nb : nullptr;
  uint8_t* r = a.rec.base ? a.rec.base + u * a.rec.stride : nullptr;
  uint32_t* po = a.plane_off ? a.plane_off + u * nb : nullptr;
  for (int64_t base = lo; base < hi; base += 4 * blockDim.x) {
    const int64_t i0 = base + 4 * static_cast<int64_t>(threadIdx.x);
    float vi[4];
    if (vv.planes) {
      // the chunk's variances into LDS in bin order, read position by
      // position (consecutive threads, consecutive positions of one head)
      const int64_t end = base + 4 * blockDim.x < hi ? base + 4 * blockDim.x : hi;
      const int64_t pos_lo = base / vv.kv;
      const uint32_t np = static_cast<uint32_t>((end - 1) / vv.kv - pos_lo + 1);
      __syncthreads();                       // the previous chunk is read
      for (uint32_t e = threadIdx.x; e < static_cast<uint32_t>(vv.kv) * np; e += blockDim.x) {
        const uint32_t h = e / np;
        const int64_t pos = pos_lo + (e - h * np);
        const int64_t i = pos * vv.kv + h;
        if (i >= base && i < end) s_var[i - base] = vv.at(static_cast<int>(h), pos, a.var_scale);
      }
      __syncthreads();
      for (int j = 0; j < 4; ++j) vi[j] = i0 + j < hi ? s_var[4 * threadIdx.x + j] : 0.f;
    } else {
      var4(vv.v, nb, vv.parts, a.var_scale, vv.vec, i0, vi);
    }
    int b[4] = {0, 0, 0, 0}, eqv[4] = {0, 0, 0, 0};
    int eq_sum = 0;
    for (int j = 0; j < 4; ++j) {
      if (i0 + j >= hi) continue;
      if (g.alloc_mode == TACT_ALLOC_UNIFORM) {
        b[j] = g.budget_bits;
      } else if (wf) {
        const uint64_t key = gain_key(vi[j]);
        b[j] = count_ge(key, tau + 1, bmax);
        eqv[j] = count_ge(key, tau, bmax) - b[j];
        eq_sum += eqv[j];
      }
    }
    if (wf) {
      if (all_ties) {
        for (int j = 0; j < 4; ++j) b[j] += eqv[j];
      } else {
        int tot_eq;
        const int ex = block_exscan(eq_sum, sh, &tot_eq);
        int64_t before = tie_carry + ex;
        for (int j = 0; j < 4; ++j) {
          int64_t avail = need - before;
          avail = avail < 0 ? 0 : avail;
          const int take = static_cast<int>(avail < eqv[j] ? avail : eqv[j]);
          b[j] += take;
          before += eqv[j];
        }
        tie_carry += tot_eq;
      }
    }
    const int bsum = b[0] + b[1] + b[2] + b[3];
    int ptot;
    const int pex = block_exscan(bsum, sh, &ptot);
    int64_t p = plane_carry + pex;
    for (int j = 0; j < 4; ++j) {
      const int64_t i = i0 + j;
      if (i < hi) {
        if (bo) bo[i] = static_cast<uint8_t>(b[j]);
        if (po) po[i] = static_cast<uint32_t>(p);
        if (a.var_out) a.var_out[u * nb + i] = vi[j];
        const float gn = sqrtf(vi[j]);
        if (a.inv_gain) a.inv_gain[u * a.var_stride + i] = gn > 0.f ? 1.0f / gn : 0.f;
        if (r) {
          reinterpret_cast<float*>(r + g.off_gains)[i] = gn;
          r[g.off_bits + i] = static_cast<uint8_t>(b[j]);
          if ((i & 63) == 0) reinterpret_cast<uint32_t*>(r + g.off_groups)[i >> 6] = static_cast<uint32_t>(p);
        }
      }
      p += b[j];
    }
    plane_carry += ptot;
  }
  if (r && blockIdx.x == 0) {
    for (int64_t k = g.off_gains + 4 * nb + threadIdx.x; k < g.off_bits; k += blockDim.x) r[k] = 0;
    for (int64_t k = g.off_bits + nb + threadIdx.x; k < g.off_groups; k += blockDim.x) r[k] = 0;
    for (int64_t k = g.off_groups + 4 * g.n_groups + threadIdx.x; k < g.off_codes; k += blockDim.x)
      r[k] = 0;
    for (int64_t k = g.off_codes + g.code_bytes + threadIdx.x; k < g.record_bytes; k += blockDim.x)
      r[k] = 0;
  }
}

// Per-bin first plane from a record (decoding side): the record's group
// index holds the first plane of every 64th bin; a thread takes four bins
// (one 4-byte load of their bit counts), so 16 lanes cover a group and scan
// it from that base.  The bit-count region is padded to 256 bytes and 4-byte
// aligned in every record, so the load past n_bins stays in the record.
__global__ __launch_bounds__(256) void k_plane_offsets(Geometry g, RecordView rec0,
                                                       uint32_t* __restrict__ out0, RecordView rec1,
                                                       uint32_t* __restrict__ out1, int64_t blocks0) {
  // blocks [0, blocks0) scan the records of rec0 into out0, the rest those of
  // rec1 into out1 (both sets of one call: the K and V records of attention)
  const bool second = blockIdx.x >= blocks0;
  const RecordView rec = second ? rec1 : rec0;
  uint32_t* plane_off = second ? out1 : out0;
  const int64_t bid = second ? blockIdx.x - blocks0 : blockIdx.x;
  const int64_t n = g.n_bins, per_unit = (n + 1023) / 1024;
  const int64_t u = bid / per_unit;
  const int64_t bin = 4 * ((bid - u * per_unit) * 256 + threadIdx.x);
  const bool live = bin < n;
  const uint8_t* r = rec.base + u * rec.stride;
  const uint32_t w = live ? *reinterpret_cast<const uint32_t*>(r + rec.off_bits + bin) : 0u;
  const int b0 = w & 255, b1 = bin + 1 < n ? (w >> 8) & 255 : 0,
            b2 = bin + 2 < n ? (w >> 16) & 255 : 0, b3 = bin + 3 < n ? w >> 24 : 0;
  const int sum = b0 + b1 + b2 + b3;
  const int seg = threadIdx.x % 16;
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    const int o = __shfl_up(incl, off, 16);
    if (seg >= off) incl += o;
  }
  if (!live) return;
  const uint32_t p0 =
      reinterpret_cast<const uint32_t*>(r + rec.off_groups)[bin >> 6] + static_cast<uint32_t>(incl - sum);
  const uint32_t p1 = p0 + b0, p2 = p1 + b1, p3 = p2 + b2;
  uint32_t* po = plane_off + u * n + bin;
  if ((n & 3) == 0) {
    *reinterpret_cast<uint4*>(po) = make_uint4(p0, p1, p2, p3);
  } else {
    po[0] = p0;
    if (bin + 1 < n) po[1] = p1;
    if (bin + 2 < n) po[2] = p2;
    if (bin + 3 < n) po[3] = p3;
  }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
template <int NP, int PRO, int EPI, int TPW>
void launch_axis_t(const AxisArgs& a, hipStream_t s) {
  const int64_t groups = a.inner / (16 * TPW);
  // about 2048 blocks (8 per CU): each wave walks several column groups so
  // that the matrix fragments are built once per wave
  const int64_t rows = a.outer * a.n_units;
  int64_t gx = (2048 + rows - 1) / rows;
  const int64_t gmax = (groups + 3) / 4;
  if (gx > gmax) gx = gmax;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL((k_axis<NP, PRO, EPI, TPW>),
                     dim3(static_cast<unsigned>(gx), static_cast<unsigned>(a.outer),
                          static_cast<unsigned>(a.n_units)),
                     dim3(256), 0, s, a);
}

template <int NP, int PRO, int EPI>
void launch_axis_tpw(const AxisArgs& a, int tpw, hipStream_t s) {
  if (tpw == 4) launch_axis_t<NP, PRO, EPI, 4>(a, s);
  else if (tpw == 8) launch_axis_t<NP, PRO, EPI, 8>(a, s);
  else launch_axis_t<NP, PRO, EPI, 16>(a, s);
}

template <int NP>
void launch_axis_np(const AxisArgs& a, int pro, int epi, int tpw, hipStream_t s) {
  if (epi == EPI_STATS) {
    if (pro == PRO_BF16) launch_axis_tpw<NP, PRO_BF16, EPI_STATS>(a, tpw, s);
    else launch_axis_tpw<NP, PRO_F32, EPI_STATS>(a, tpw, s);
  } else if (epi == EPI_QUANT) {
    if (pro == PRO_BF16) launch_axis_tpw<NP, PRO_BF16, EPI_QUANT>(a, tpw, s);
    else launch_axis_tpw<NP, PRO_F32, EPI_QUANT>(a, tpw, s);
  } else if (epi == EPI_F32) {
    // bf16 rows: 8 elements (16 bytes) per lane when the row holds whole
    // 128-column groups, else 4
    if (pro == PRO_BF16 && a.inner % 128 == 0) launch_axis_t<NP, PRO_BF16, EPI_F32, 8>(a, s);
    else if (pro == PRO_BF16) launch_axis_t<NP, PRO_BF16, EPI_F32, 4>(a, s);
    else if (pro == PRO_F32) launch_axis_t<NP, PRO_F32, EPI_F32, 4>(a, s);
    else launch_axis_t<NP, PRO_DEQUANT, EPI_F32, 4>(a, s);
  } else {
    if (pro == PRO_F32) launch_axis_t<NP, PRO_F32, EPI_BF16, 4>(a, s);
    else if (pro == PRO_BF16 && a.inner % 128 == 0) launch_axis_t<NP, PRO_BF16, EPI_BF16, 8>(a, s);
    else if (pro == PRO_BF16) launch_axis_t<NP, PRO_BF16, EPI_BF16, 4>(a, s);
    else launch_axis_t<NP, PRO_DEQUANT, EPI_BF16, 4>(a, s);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// host-facing launchers (declared in tact_internal.h)
// ---------------------------------------------------------------------------
void launch_dct_tables(const Geometry& g, float* tab, hipStream_t s, int identity) {
  if (identity < 0) identity = g.axes == 0 ? 1 : 0;
  hipLaunchKernelGGL(k_dct_tables, dim3(3), dim3(256), 0, s, tab, g.S, g.H, g.W, identity);
}

// axis: 0 = S, 1 = H, 2 = W
static void axis_shape(const Geometry& g, int axis, int* N, int64_t* outer, int64_t* inner) {
  const int64_t C = static_cast<int64_t>(g.kv_heads) * g.head_dim;
  if (axis == 0) {
    *N = g.S; *outer = 1; *inner = static_cast<int64_t>(g.H) * g.W * C;
  } else if (axis == 1) {
    *N = g.H; *outer = g.S; *inner = static_cast<int64_t>(g.W) * C;
  } else {
    *N = g.W; *outer = static_cast<int64_t>(g.S) * g.H; *inner = C;
  }
}

void launch_axis(const Geometry& g, int64_t n_units, int axis, int inverse, int pro, int epi,
                 const void* in, int64_t in_stride, void* out, int64_t out_stride,
                 const float* tab, float* var, const float* inv_gain, int64_t var_stride,
                 RecordView rec, const uint32_t* plane_off, hipStream_t s, bool rot_in,
                 bool rot_out) {
  AxisArgs a;
  a.in = in;
  a.in_ustride = in_stride;
  a.out = out;
  a.out_ustride = out_stride;
  a.tab = tab + axis * 4096;
  a.inverse = inverse;
  axis_shape(g, axis, &a.N, &a.outer, &a.inner);
  a.n_units = n_units;
  a.head_dim = g.head_dim;
  a.kv_heads = g.kv_heads;
  a.C = static_cast<int64_t>(g.kv_heads) * g.head_dim;
  a.n_bins = g.n_bins;
  a.total_bits = g.total_bits;
  a.max_bits = g.max_bits;
  a.var = var;
  a.inv_gain = inv_gain;
  a.var_stride = var_stride;
  a.rec = rec;
  a.plane_off = plane_off;
  a.rotate = g.rotation == TACT_ROTATION_HADAMARD;
  a.quant = g.quantizer;
  a.rot_in = rot_in && a.rotate && pro == PRO_F32 && (epi == EPI_F32 || epi == EPI_BF16);
  a.rot_out = rot_out && a.rotate && pro != PRO_DEQUANT && epi == EPI_F32;
  const int tpw = (epi == EPI_STATS || epi == EPI_QUANT) ? g.head_dim / 16 : 4;
  if (a.N <= 16) launch_axis_np<16>(a, pro, epi, tpw, s);
  else if (a.N <= 32) launch_axis_np<32>(a, pro, epi, tpw, s);
  else launch_axis_np<64>(a, pro, epi, tpw, s);
}


// Blocks of a persistent launch: the device's resident capacity for this
// kernel (compute units x blocks per unit), at most `work`, at least 1.
static int64_t persistent_blocks(const void* fn, int threads, size_t lds, int64_t work) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int64_t n = static_cast<int64_t>(cus) * per_cu;
  if (n > work) n = work;
  return n < 1 ? 1 : n;
}

// Grid of the XCD-aware plane walk: a whole number of XCD rounds, at least
// one block per XCD (blocks whose list is empty exit at once).
static int64_t xcd_grid(int64_t n) {
  return n < kXcds ? kXcds : n / kXcds * kXcds;
}

bool plane_supported(const Geometry& g) {
  return (g.axes & 6) == 6 && g.H <= 32 && g.W <= 32 &&
         static_cast<int64_t>(g.H) * g.W * 64 * 4 <= 150 * 1024;
}

void launch_plane(const Geometry& g, int64_t n_units, int mode, const float* in, float* out,
                  int64_t ustride, const float* tab, float* var_part, int64_t var_stride,
                  RecordView rec, const uint32_t* plane_off, hipStream_t s) {
  PlaneArgs a;
  a.in = in;
  a.out = out;
  a.ustride = ustride;
  a.tab = tab;
  a.S = g.S;
  a.H = g.H;
  a.W = g.W;
  a.C = static_cast<int64_t>(g.kv_heads) * g.head_dim;
  a.head_dim = g.head_dim;
  a.kv_heads = g.kv_heads;
  a.n_bins = g.n_bins;
  a.total_bits = g.total_bits;
  a.max_bits = g.max_bits;
  a.var_part = var_part;
  a.parts = g.head_dim / 64;
  a.var_stride = var_stride;
  a.rec = rec;
  a.plane_off = plane_off;
  a.n_units = n_units;
  const int64_t n_planes = n_units * g.S * (a.C / 64);
  const int span = g.H > g.W ? g.H : g.W;
  const int waves = (mode == MODE_DEQUANT && span > 16 && span <= 24) ? kDecodeWaves : kPlaneWaves;
  const dim3 block(64 * waves);
  const bool h16 = g.H <= 16, w16 = g.W <= 16;
  // the decode pass pads rows shorter than its staging of the 16 or 32 K
  // rows (decode_stage_bytes)
  int rw = g.W;
  if (mode == MODE_DEQUANT) {
    const int nk = w16 ? 16 : 32;
    const int need = (decode_stage_bytes(nk) + 255) / 256;
    if (rw < need) rw = need;
  }
  const size_t lds = static_cast<size_t>(g.H) * rw * 64 * sizeof(float);
  // the plane needs more dynamic LDS than the default limit
  // persistent grid: as many blocks as the device holds at once
#define TACT_PLANE_ONE(NH, NW, M, SL, WV)                                                       \
  do {                                                                                          \
    const void* fn = reinterpret_cast<const void*>(&k_plane<NH, NW, M, SL, WV>);                \
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,                   \
                              static_cast<int>(lds));                                           \
    const dim3 grid(static_cast<unsigned>(xcd_grid(persistent_blocks(fn, 64 * waves, lds, n_planes)))); \
    hipLaunchKernelGGL((k_plane<NH, NW, M, SL, WV>), grid, block, lds, s, a);                   \
  } while (0)
#define TACT_PLANE_SL(NH, NW, SL)                                                               \
  do {                                                                                          \
    if (mode == MODE_STATS) TACT_PLANE_ONE(NH, NW, MODE_STATS, SL, kPlaneWaves);                \
    else TACT_PLANE_ONE(NH, NW, MODE_DEQUANT, SL, kPlaneWaves);                                 \
  } while (0)
#define TACT_PLANE(NH, NW)                                                                      \
  do {                                                                                          \
    if (slots <= 2) TACT_PLANE_SL(NH, NW, 2);                                                   \
    else if (slots == 3) TACT_PLANE_SL(NH, NW, 3);                                              \
    else TACT_PLANE_SL(NH, NW, 4);                                                              \
  } while (0)
  const int slots = (span + kPlaneWaves - 1) / kPlaneWaves;
  if (waves == kDecodeWaves) {             // decode, 17..24 rows or columns
    if (h16) TACT_PLANE_ONE(16, 32, MODE_DEQUANT, 2, kDecodeWaves);
    else if (w16) TACT_PLANE_ONE(32, 16, MODE_DEQUANT, 2, kDecodeWaves);
    else TACT_PLANE_ONE(32, 32, MODE_DEQUANT, 2, kDecodeWaves);
  } else if (h16 && w16) TACT_PLANE_SL(16, 16, 2);
  else if (h16) TACT_PLANE(16, 32);
  else if (w16) TACT_PLANE(32, 16);
  else TACT_PLANE(32, 32);
#undef TACT_PLANE
#undef TACT_PLANE_SL
#undef TACT_PLANE_ONE
}

// Bins per allocation workgroup: about 16K, at most kAllocMaxSlices slices
// per unit, a multiple of the final pass's chunk and of 4 kv_heads (a slice
// is then whole positions of every head, a multiple of 4 of them).
int64_t alloc_slice(const Geometry& g) {
  int64_t want = (g.n_bins + kAllocMaxSlices - 1) / kAllocMaxSlices;
  if (want < 16384) want = 16384;
  int64_t a = kAllocChunk, b = 4 * static_cast<int64_t>(g.kv_heads);
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  const int64_t al = kAllocChunk / a * (4 * static_cast<int64_t>(g.kv_heads));   // lcm
  return (want + al - 1) / al * al;
}

void launch_allocate2(const Geometry& g, int64_t n_units, const float* var, int64_t var_stride,
                      int parts, float var_scale, uint8_t* bits_out, RecordView rec,
                      uint32_t* plane_off, float* inv_gain, void* scratch, hipStream_t s,
                      bool planes, float* var_out) {
  AllocArgs a;
  a.g = g;
  a.var = var;
  a.var_stride = var_stride;
  a.parts = parts;
  a.var_scale = var_scale;
  a.planes = planes ? 1 : 0;
  a.scratch = static_cast<uint8_t*>(scratch);
  a.slice = alloc_slice(g);
  a.bits_out = bits_out;
  a.rec = rec;
  a.plane_off = plane_off;
  a.inv_gain = inv_gain;
  a.var_out = var_out;
  const dim3 grid(static_cast<unsigned>((g.n_bins + a.slice - 1) / a.slice),
                  static_cast<unsigned>(n_units));
  const dim3 block(kAllocThreads);
  if (g.alloc_mode == TACT_ALLOC_WATERFILL && g.total_bits > 0) {
    hipLaunchKernelGGL(k_alloc_clear, dim3(static_cast<unsigned>(n_units)), dim3(256), 0, s, a.scratch);
    hipLaunchKernelGGL(k_alloc_hist<1>, grid, block, 0, s, a);
    hipLaunchKernelGGL(k_alloc_hist<2>, grid, block, 0, s, a);
    hipLaunchKernelGGL(k_alloc_hist<3>, grid, block, 0, s, a);
  }
  hipLaunchKernelGGL(k_alloc_count, grid, block, 0, s, a);
  hipLaunchKernelGGL(k_alloc_write, grid, block, 0, s, a);
}

void launch_plane_offsets(const Geometry& g, int64_t n_units, RecordView rec, uint32_t* plane_off,
                          hipStream_t s, const RecordView* rec2, uint32_t* plane_off2) {
  const int64_t blocks = (g.n_bins + 1023) / 1024 * n_units;
  const int64_t total = rec2 ? 2 * blocks : blocks;
  hipLaunchKernelGGL(k_plane_offsets, dim3(static_cast<unsigned>(total)), dim3(256), 0, s, g, rec,
                     plane_off, rec2 ? *rec2 : rec, rec2 ? plane_off2 : plane_off, blocks);
}

}  // namespace tact
