// gfx950 kernels of the TACT-KV codec (page "TACT-KV: Tri-Axis Cosine
// Transform for Compressing Volumetric KV Caches in Medical VLMs", section
// "Methodology in Plain English", stages 2-4 and the decoding paragraph).
//
// Straightforward first path: one kernel per step, fp32 coefficients held
// in the workspace between steps.
//   k_dct_axis      one axis of the separable DCT-II / DCT-III; a thread owns
//                   one column along the axis (coalesced over the trailing,
//                   contiguous dimensions) and runs in place.
//   k_bin_variance  one wave64 per bin, fixed shuffle tree (deterministic).
//   k_allocate      one 1024-thread workgroup per unit: exact bisection of
//                   the water level over the integer image of the fp64
//                   marginal gains, then the tie order as a block scan.
//   k_quantize      one wave64 per bin: fp32 decision, one ballot per
//                   bit-plane gives whole 64-bit code words.
//   k_unpack        one wave64 per bin: bit-planes back to codes, dequantize.
#include <hip/hip_runtime.h>

#include "tact_internal.h"

namespace tact {

#include "codebook_device.h"

const float kHostLevels[TACT_CODEBOOK_LEVELS] = {TACT_CODEBOOK_LEVEL_VALUES};
const float kHostThresholds[TACT_CODEBOOK_THRESHOLDS] = {TACT_CODEBOOK_THRESHOLD_VALUES};
static const float kHostUniformLevels[TACT_CODEBOOK_LEVELS] = {TACT_UNIFORM_LEVEL_VALUES};
static const float kHostUniformThresholds[TACT_CODEBOOK_THRESHOLDS] = {TACT_UNIFORM_THRESHOLD_VALUES};
static const float kHostNfLevels[TACT_CODEBOOK_LEVELS] = {TACT_NF_LEVEL_VALUES};
static const float kHostNfThresholds[TACT_CODEBOOK_THRESHOLDS] = {TACT_NF_THRESHOLD_VALUES};
const float* const kHostLevelsQ[3] = {kHostLevels, kHostUniformLevels, kHostNfLevels};
const float* const kHostThresholdsQ[3] = {kHostThresholds, kHostUniformThresholds, kHostNfThresholds};

namespace {

constexpr int kWave = 64;

__device__ __forceinline__ float load_as_float(const float* p) { return *p; }
__device__ __forceinline__ float load_as_float(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
__device__ __forceinline__ void store_from_float(float* p, float v) { *p = v; }
// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ void store_from_float(uint16_t* p, float v) {
  const uint32_t u = __float_as_uint(v);
  *p = static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// Stage 2: one axis of the separable orthonormal DCT.
// Column c = (outer o, inner b); element n of the column sits at
// o*N*inner + n*inner + b.  Forward: y_k = sum_n C[k][n] x_n;
// inverse: x_n = sum_k C[k][n] y_k, C[k][n] = a_k cos(pi (2n+1) k / 2N).
// ---------------------------------------------------------------------------
template <int NMAX, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void k_dct_axis(
    const TIn* __restrict__ in, int64_t in_stride, TOut* __restrict__ out,
    int64_t out_stride, int64_t n_outer, int N, int64_t inner, int inverse) {
  __shared__ float cm[NMAX * NMAX];
  for (int t = threadIdx.x; t < N * N; t += blockDim.x) {
    const int r = t / N, s = t % N;          // output r, input s
    const int k = inverse ? s : r;
    const int n = inverse ? r : s;
    const double a = (k == 0) ? sqrt(1.0 / N) : sqrt(2.0 / N);
    cm[r * NMAX + s] = static_cast<float>(a * cospi((2.0 * n + 1.0) * k / (2.0 * N)));
  }
  __syncthreads();
  const int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (col >= n_outer * inner) return;
  const int64_t o = col / inner, b = col - o * inner;
  const int64_t base = o * N * inner + b;
  const TIn* src = in + static_cast<int64_t>(blockIdx.y) * in_stride + base;
  TOut* dst = out + static_cast<int64_t>(blockIdx.y) * out_stride + base;
  float x[NMAX];
#pragma unroll
  for (int n = 0; n < NMAX; ++n) x[n] = (n < N) ? load_as_float(src + n * inner) : 0.f;
#pragma unroll
  for (int r = 0; r < NMAX; ++r) {
    if (r < N) {
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < NMAX; ++s)
        if (s < N) acc = fmaf(cm[r * NMAX + s], x[s], acc);
      store_from_float(dst + r * inner, acc);
    }
  }
}

template <typename TIn, typename TOut>
void dct_axis_launch(const Geometry& g, int64_t n_units, int axis, int inverse,
                     const void* in, int64_t in_stride, void* out,
                     int64_t out_stride, hipStream_t stream) {
  const int64_t C = static_cast<int64_t>(g.kv_heads) * g.head_dim;
  int N;
  int64_t outer, inner;
  if (axis == 0) {
    N = g.S; outer = 1; inner = static_cast<int64_t>(g.H) * g.W * C;
  } else if (axis == 1) {
    N = g.H; outer = g.S; inner = static_cast<int64_t>(g.W) * C;
  } else {
    N = g.W; outer = static_cast<int64_t>(g.S) * g.H; inner = C;
  }
  const int64_t cols = outer * inner;
  dim3 grid(static_cast<unsigned>((cols + 255) / 256), static_cast<unsigned>(n_units));
  auto* i = static_cast<const TIn*>(in);
  auto* o = static_cast<TOut*>(out);
  if (N <= 8)
    hipLaunchKernelGGL((k_dct_axis<8, TIn, TOut>), grid, dim3(256), 0, stream, i, in_stride, o, out_stride, outer, N, inner, inverse);
  else if (N <= 16)
    hipLaunchKernelGGL((k_dct_axis<16, TIn, TOut>), grid, dim3(256), 0, stream, i, in_stride, o, out_stride, outer, N, inner, inverse);
  else if (N <= 32)
    hipLaunchKernelGGL((k_dct_axis<32, TIn, TOut>), grid, dim3(256), 0, stream, i, in_stride, o, out_stride, outer, N, inner, inverse);
  else
    hipLaunchKernelGGL((k_dct_axis<64, TIn, TOut>), grid, dim3(256), 0, stream, i, in_stride, o, out_stride, outer, N, inner, inverse);
}

void dct_axis_dispatch(const Geometry& g, int64_t n_units, int axis, int inverse,
                       const void* in, int in_dtype, int64_t in_stride,
                       void* out, int out_dtype, int64_t out_stride,
                       hipStream_t stream) {
  if (in_dtype == TACT_BF16 && out_dtype == TACT_F32)
    dct_axis_launch<uint16_t, float>(g, n_units, axis, inverse, in, in_stride, out, out_stride, stream);
  else if (in_dtype == TACT_F32 && out_dtype == TACT_BF16)
    dct_axis_launch<float, uint16_t>(g, n_units, axis, inverse, in, in_stride, out, out_stride, stream);
  else if (in_dtype == TACT_BF16 && out_dtype == TACT_BF16)
    dct_axis_launch<uint16_t, uint16_t>(g, n_units, axis, inverse, in, in_stride, out, out_stride, stream);
  else
    dct_axis_launch<float, float>(g, n_units, axis, inverse, in, in_stride, out, out_stride, stream);
}

// ---------------------------------------------------------------------------
// Stage 3a: per-bin second moment over head_dim.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__global__ __launch_bounds__(256) void k_bin_variance(const float* __restrict__ coef,
                                                      float* __restrict__ var,
                                                      int64_t total_bins, int d) {
  const int64_t bin = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (bin >= total_bins) return;
  const float* c = coef + bin * d;
  float s = 0.f;
  for (int r = 0; r < d / kWave; ++r) {
    const float v = c[r * kWave + lane];
    s = fmaf(v, v, s);
  }
  s = wave_sum(s);
  if (lane == 0) var[bin] = s * (1.0f / static_cast<float>(d));
}

// ---------------------------------------------------------------------------
// Stage 3b: reverse water-filling on the exact key set.
// The marginal gain of bin i's k-th bit is var_i * 4^-(k-1).  In fp64 that
// value is var_i with the exponent lowered by 2(k-1), so its bit pattern is
// K_i - (k-1) * 2^53 with K_i the pattern of (double)var_i; patterns of
// positive doubles order like their values.  Bins with zero variance have
// gain 0 for every k (pattern 0, below every positive gain).  The water
// level is found by bisection over these integers: tau = the largest value
// with count(gain >= tau) >= T, which is the T-th largest gain.  Bins get
// every bit whose gain exceeds tau; bits whose gain equals tau go to the
// lowest bin indices first (k ascending within a bin) until T is reached.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t gain_key(float v) {
  return v > 0.f ? __double_as_longlong(static_cast<double>(v)) : 0;
}

__device__ __forceinline__ int count_ge(int64_t key, int64_t tau, int bmax) {
  if (key == 0) return tau <= 0 ? bmax : 0;
  const int64_t diff = key - tau;
  if (diff < 0) return 0;
  const int64_t q = (diff >> 53) + 1;
  return q > bmax ? bmax : static_cast<int>(q);
}

constexpr int kAllocThreads = 1024;

template <typename T>
__device__ T block_sum(T v, T* red) {
  // red: kAllocThreads / 64 slots
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  T t = 0;
  for (int i = 0; i < static_cast<int>(blockDim.x) / kWave; ++i) t += red[i];
  return t;
}

template <typename T>
__device__ T block_max(T v, T* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const T o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  T t = red[0];
  for (int i = 1; i < static_cast<int>(blockDim.x) / kWave; ++i) t = red[i] > t ? red[i] : t;
  return t;
}

// Exclusive prefix sum over the block (thread order); returns the block total
// through *total.
__device__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  __syncthreads();
  if (lane == kWave - 1) scratch[w] = incl;
  __syncthreads();
  int before = 0, all = 0;
  const int nw = static_cast<int>(blockDim.x) / kWave;
  for (int i = 0; i < nw; ++i) {
    if (i < w) before += scratch[i];
    all += scratch[i];
  }
  *total = all;
  return before + incl - v;
}

// Writes gains/bits/group index and zeroes the record padding; `bits_of(i)`
// gives bin i's bits, the gains come from `gain_of(i)`.  All threads call.
template <typename BitsF, typename GainF>
__device__ void write_header(const Geometry& g, uint8_t* rec, BitsF bits_of,
                             GainF gain_of, int* scratch) {
  float* gains = reinterpret_cast<float*>(rec + g.off_gains);
  uint8_t* bits = rec + g.off_bits;
  uint32_t* groups = reinterpret_cast<uint32_t*>(rec + g.off_groups);
  int64_t carry = 0;
  for (int64_t base = 0; base < g.n_bins; base += blockDim.x) {
    const int64_t i = base + threadIdx.x;
    const int b = (i < g.n_bins) ? bits_of(i) : 0;
    int tot;
    const int ex = block_exclusive_scan(b, scratch, &tot);
    if (i < g.n_bins) {
      gains[i] = gain_of(i);
      bits[i] = static_cast<uint8_t>(b);
      if ((i & 63) == 0) groups[i >> 6] = static_cast<uint32_t>(carry + ex);
    }
    carry += tot;
  }
  // zero the alignment padding of every region
  auto zero = [&](int64_t from, int64_t to) {
    for (int64_t k = from + threadIdx.x; k < to; k += blockDim.x) rec[k] = 0;
  };
  zero(g.off_gains + 4 * g.n_bins, g.off_bits);
  zero(g.off_bits + g.n_bins, g.off_groups);
  zero(g.off_groups + 4 * g.n_groups, g.off_codes);
  zero(g.off_codes + g.code_bytes, g.record_bytes);
}

__global__ __launch_bounds__(kAllocThreads) void k_allocate(
    Geometry g, const float* __restrict__ var, uint8_t* __restrict__ bits_out,
    RecordView rec) {
  __shared__ int64_t red64[kAllocThreads / kWave];
  __shared__ int scratch[kAllocThreads / kWave];
  const int64_t u = blockIdx.x;
  const float* v = var + u * g.n_bins;
  const int bmax = g.max_bits;
  const int64_t T = g.total_bits;

  int64_t tau = 0;
  int64_t need = 0;
  if (g.alloc_mode == TACT_ALLOC_WATERFILL && T > 0) {
    int64_t kmax = 0;
    for (int64_t i = threadIdx.x; i < g.n_bins; i += blockDim.x) {
      const int64_t k = gain_key(v[i]);
      kmax = k > kmax ? k : kmax;
    }
    kmax = block_max(kmax, red64);
    int64_t lo = 0, hi = kmax + 1;   // count_ge(lo) >= T > count_ge(hi)
    while (hi - lo > 1) {
      const int64_t mid = lo + (hi - lo) / 2;
      int64_t c = 0;
      for (int64_t i = threadIdx.x; i < g.n_bins; i += blockDim.x)
        c += count_ge(gain_key(v[i]), mid, bmax);
      c = block_sum(c, red64);
      if (c >= T) lo = mid; else hi = mid;
    }
    tau = lo;
    int64_t gt = 0;
    for (int64_t i = threadIdx.x; i < g.n_bins; i += blockDim.x)
      gt += count_ge(gain_key(v[i]), tau + 1, bmax);
    need = T - block_sum(gt, red64);
  }

  // bits of every bin: strictly-above-tau bits plus tied bits in bin order
  uint8_t* bo = bits_out ? bits_out + u * g.n_bins : nullptr;
  uint8_t* r = rec.base ? rec.base + u * rec.stride : nullptr;
  float* gains = r ? reinterpret_cast<float*>(r + g.off_gains) : nullptr;
  uint8_t* rbits = r ? r + g.off_bits : nullptr;
  uint32_t* groups = r ? reinterpret_cast<uint32_t*>(r + g.off_groups) : nullptr;
  int64_t tie_carry = 0, plane_carry = 0;
  for (int64_t base = 0; base < g.n_bins; base += blockDim.x) {
    const int64_t i = base + threadIdx.x;
    int b = 0;
    float vi = 0.f;
    int eq = 0, gtb = 0;
    if (i < g.n_bins) {
      vi = v[i];
      if (g.alloc_mode == TACT_ALLOC_UNIFORM) {
        gtb = g.budget_bits;
      } else if (T > 0) {
        const int64_t k = gain_key(vi);
        gtb = count_ge(k, tau + 1, bmax);
        eq = count_ge(k, tau, bmax) - gtb;
      }
    }
    int tot;
    const int ex = block_exclusive_scan(eq, scratch, &tot);
    int64_t avail = need - (tie_carry + ex);
    avail = avail < 0 ? 0 : avail;
    b = gtb + static_cast<int>(avail < eq ? avail : eq);
    tie_carry += tot;
    int ptot;
    const int pex = block_exclusive_scan(b, scratch, &ptot);
    if (i < g.n_bins) {
      if (bo) bo[i] = static_cast<uint8_t>(b);
      if (r) {
        gains[i] = sqrtf(vi);
        rbits[i] = static_cast<uint8_t>(b);
        if ((i & 63) == 0) groups[i >> 6] = static_cast<uint32_t>(plane_carry + pex);
      }
    }
    plane_carry += ptot;
  }
  if (r) {
    auto zero = [&](int64_t from, int64_t to) {
      for (int64_t k = from + threadIdx.x; k < to; k += blockDim.x) r[k] = 0;
    };
    zero(g.off_gains + 4 * g.n_bins, g.off_bits);
    zero(g.off_bits + g.n_bins, g.off_groups);
    zero(g.off_groups + 4 * g.n_groups, g.off_codes);
    zero(g.off_codes + g.code_bytes, g.record_bytes);
  }
}

__global__ __launch_bounds__(kAllocThreads) void k_header(Geometry g,
                                                          const float* __restrict__ gains,
                                                          const uint8_t* __restrict__ bits,
                                                          RecordView rec) {
  __shared__ int scratch[kAllocThreads / kWave];
  const int64_t u = blockIdx.x;
  const float* gu = gains + u * g.n_bins;
  const uint8_t* bu = bits + u * g.n_bins;
  write_header(
      g, rec.base + u * rec.stride, [&](int64_t i) { return static_cast<int>(bu[i]); },
      [&](int64_t i) { return gu[i]; }, scratch);
}

// ---------------------------------------------------------------------------
// Stage 4: gain-shape quantization and bit-plane packing.
// ---------------------------------------------------------------------------
// First bit-plane of bin i: group index plus the bits of the bins of its
// 64-bin group that precede it (wave-wide sum).
__device__ __forceinline__ int64_t plane_offset(const uint8_t* bits,
                                                const uint32_t* groups, int64_t i,
                                                int64_t n_bins, int lane) {
  const int64_t g0 = i & ~static_cast<int64_t>(63);
  const int64_t k = g0 + lane;
  int v = (k < i) ? bits[k] : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return static_cast<int64_t>(groups[i >> 6]) + v;
}

// Number of the 2^b - 1 ascending fp32 thresholds that are <= u.
__device__ __forceinline__ int cell_index(float u, int b) {
  const float* t = c_thresholds + ((1 << b) - b - 1);
  int pos = 0;
  for (int step = 1 << (b - 1); step >= 1; step >>= 1)
    if (t[pos + step - 1] <= u) pos += step;
  return pos;
}

__global__ __launch_bounds__(256) void k_quantize(Geometry g, int64_t n_units,
                                                  const float* __restrict__ coef,
                                                  RecordView rec) {
  const int64_t gb = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (gb >= n_units * g.n_bins) return;
  const int64_t u = gb / g.n_bins, i = gb - u * g.n_bins;
  uint8_t* r = rec.base + u * rec.stride;
  const uint8_t* bits = r + rec.off_bits;
  const int b = bits[i];
  if (b == 0 || b > g.max_bits) return;
  const int64_t p0 = plane_offset(bits, reinterpret_cast<const uint32_t*>(r + rec.off_groups),
                                  i, g.n_bins, lane);
  if (p0 < 0 || p0 + b > g.total_bits) return;   // bits that overrun the budget
  const float gain = reinterpret_cast<const float*>(r + rec.off_gains)[i];
  const float inv = gain > 0.f ? 1.0f / gain : 0.f;
  uint64_t* words = reinterpret_cast<uint64_t*>(r + rec.off_codes);
  const int wpp = g.head_dim / kWave;                 // words per plane
  const float* c = coef + gb * g.head_dim;
  for (int w = 0; w < wpp; ++w) {
    const float uq = c[w * kWave + lane] * inv;
    const int code = cell_index(uq, b);
    for (int q = 0; q < b; ++q) {
      const uint64_t word = __ballot((code >> q) & 1);
      if (lane == 0) words[(p0 + q) * wpp + w] = word;
    }
  }
}

__global__ __launch_bounds__(256) void k_unpack(Geometry g, int64_t n_units, RecordView rec,
                                                uint8_t* __restrict__ codes_out,
                                                float* __restrict__ coef_out) {
  const int64_t gb = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (gb >= n_units * g.n_bins) return;
  const int64_t u = gb / g.n_bins, i = gb - u * g.n_bins;
  const uint8_t* r = rec.base + u * rec.stride;
  const uint8_t* bits = r + rec.off_bits;
  int b = bits[i];
  const int wpp = g.head_dim / kWave;
  int64_t p0 = 0;
  if (b > 0 && b <= g.max_bits) {
    p0 = plane_offset(bits, reinterpret_cast<const uint32_t*>(r + rec.off_groups), i,
                      g.n_bins, lane);
    if (p0 < 0 || p0 + b > g.total_bits) b = 0;   // malformed record: emit zeros
  } else {
    b = 0;
  }
  if (b == 0) {
    for (int w = 0; w < wpp; ++w) {
      if (codes_out) codes_out[gb * g.head_dim + w * kWave + lane] = 0;
      if (coef_out) coef_out[gb * g.head_dim + w * kWave + lane] = 0.f;
    }
    return;
  }
  const float gain = reinterpret_cast<const float*>(r + rec.off_gains)[i];
  const uint64_t* words = reinterpret_cast<const uint64_t*>(r + rec.off_codes);
  const float* lv = c_levels + ((1 << b) - 2);
  for (int w = 0; w < wpp; ++w) {
    int code = 0;
    for (int q = 0; q < b; ++q)
      code |= static_cast<int>((words[(p0 + q) * wpp + w] >> lane) & 1u) << q;
    if (codes_out) codes_out[gb * g.head_dim + w * kWave + lane] = static_cast<uint8_t>(code);
    if (coef_out) coef_out[gb * g.head_dim + w * kWave + lane] = gain * lv[code];
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
void launch_dct3(const Geometry& g, int64_t n_units, int inverse, const void* in,
                 int in_dtype, int64_t in_stride, void* out, int out_dtype,
                 int64_t out_stride, float* work, hipStream_t stream) {
  int order[3], m = 0;
  const int fwd[3] = {0, 1, 2}, inv[3] = {2, 1, 0};
  for (int j = 0; j < 3; ++j) {
    const int a = inverse ? inv[j] : fwd[j];
    if (g.axes & (1 << a)) order[m++] = a;
  }
  const int64_t n = g.n_entries;
  if (out_dtype == TACT_F32) {
    // first pass in -> out, the rest in place in out
    for (int j = 0; j < m; ++j) {
      if (j == 0)
        dct_axis_dispatch(g, n_units, order[j], inverse, in, in_dtype, in_stride, out,
                          TACT_F32, out_stride, stream);
      else
        dct_axis_dispatch(g, n_units, order[j], inverse, out, TACT_F32, out_stride, out,
                          TACT_F32, out_stride, stream);
    }
  } else {
    // fp32 work buffer (may alias in): all passes but the last in place in
    // work, the last one work -> out
    const void* src = in;
    int src_dtype = in_dtype;
    int64_t src_stride = in_stride;
    for (int j = 0; j < m; ++j) {
      if (j + 1 < m) {
        dct_axis_dispatch(g, n_units, order[j], inverse, src, src_dtype, src_stride, work,
                          TACT_F32, n, stream);
        src = work;
        src_dtype = TACT_F32;
        src_stride = n;
      } else {
        dct_axis_dispatch(g, n_units, order[j], inverse, src, src_dtype, src_stride, out,
                          out_dtype, out_stride, stream);
      }
    }
  }
}

void launch_bin_variance(const Geometry& g, int64_t n_units, const float* coef,
                         float* var, hipStream_t stream) {
  const int64_t total = n_units * g.n_bins;
  hipLaunchKernelGGL(k_bin_variance, dim3(static_cast<unsigned>((total + 3) / 4)), dim3(256),
                     0, stream, coef, var, total, g.head_dim);
}

void launch_allocate(const Geometry& g, int64_t n_units, const float* var,
                     uint8_t* bits_out, RecordView rec, hipStream_t stream) {
  hipLaunchKernelGGL(k_allocate, dim3(static_cast<unsigned>(n_units)), dim3(kAllocThreads), 0,
                     stream, g, var, bits_out, rec);
}

void launch_header(const Geometry& g, int64_t n_units, const float* gains,
                   const uint8_t* bits, RecordView rec, hipStream_t stream) {
  hipLaunchKernelGGL(k_header, dim3(static_cast<unsigned>(n_units)), dim3(kAllocThreads), 0,
                     stream, g, gains, bits, rec);
}

void launch_quantize(const Geometry& g, int64_t n_units, const float* coef,
                     RecordView rec, hipStream_t stream) {
  const int64_t total = n_units * g.n_bins;
  hipLaunchKernelGGL(k_quantize, dim3(static_cast<unsigned>((total + 3) / 4)), dim3(256), 0,
                     stream, g, n_units, coef, rec);
}

void launch_unpack(const Geometry& g, int64_t n_units, RecordView rec, uint8_t* codes_out,
                   float* coef_out, hipStream_t stream) {
  const int64_t total = n_units * g.n_bins;
  hipLaunchKernelGGL(k_unpack, dim3(static_cast<unsigned>((total + 3) / 4)), dim3(256), 0,
                     stream, g, n_units, rec, codes_out, coef_out);
}

}  // namespace tact
