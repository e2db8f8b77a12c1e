// Decoding fused into attention (page "TACT-KV: Tri-Axis Cosine Transform
// for Compressing Volumetric KV Caches in Medical VLMs", "Methodology in Plain
// English", the decoding paragraph): one decoding query per query head
// attends over the visual tokens of a unit pair (the K and the V record of one
// layer and sequence) without reconstructing K or V.
//
// The inverse 3-D DCT is linear and orthonormal.  With c_f the decoded
// (unrotated) coefficient vector of frequency bin f of a head and B the
// inverse transform, token t holds k_t = sum_f B[t, f] c_f, so
//   scores:  q . k_t = IDCT3(s)[t],   s_f = q . c_f = (R q) . c'_f,
//   output:  sum_t p_t v_t = sum_f DCT3(p)[f] c_f = R^T sum_f DCT3(p)[f] c'_f,
// where c'_f = g_f * level(code) is the decoded vector in the rotated frame
// (R is the quantizer's rotation).  Only coded bins contribute.  Per unit
// pair, kv head and query head the kernels compute
//   k_att_qrot   q' = scale * R q;
//   k_att_proj   s_f = g_f * sum_j level_j * q'_j over the K record's bins
//                (lane = bin, the codes read straight from the bit planes);
//   k_att_frags  the DCT tables as split fp16 MFMA fragments (once a call);
//   k_att_field  scores = IDCT3(s) in LDS on the matrix cores, the softmax,
//                lse, P = DCT3(p);
//   k_att_out    partial sums of P_f * level * g over the V record's bins
//                (lane = channel), per chunk of bins;
//   k_att_final  the sum over chunks and R^T, into the output.
// The field of one query head (S * H * W fp32) lives in LDS, so S * H * W is
// capped (the host checks it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tact_internal.h"

namespace tact {

#include "codebook_device.h"
#include "tact_rotation.h"

namespace {

constexpr int kWave = 64;

#include "tact_mfma_ops.h"
#include "tact_bitplanes.h"
// raw buffer descriptor (gfx9 word 3): loads past its byte range return 0
constexpr int kBufWord3 = 0x00020000;
constexpr int kPastBuffer = 0x7FFFFFF0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t att_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufWord3);
}
constexpr int kChunk = 256;       // bins per wave in k_att_out
constexpr int kFieldThreads = 768;

struct AttArgs {
  RecordView krec, vrec;
  const uint32_t* kpoff;          // first plane of each bin, [pair][bin]
  const uint32_t* vpoff;
  const float* q;                 // [pair][q_heads][head_dim]
  float scale;
  float* qrot;                    // [pair][q_heads][head_dim]
  float* field;                   // [pair][q_heads][S*H*W]
  float* partial;                 // [pair][kv_heads][chunk][rep][head_dim]
  float* out;                     // [pair][q_heads][head_dim]
  float* lse;                     // [pair][q_heads]
  const float* tab;               // DCT-II matrices [3][64][64]
  uint4* frags;                   // their split fp16 MFMA fragments
  int S, H, W, kv_heads, head_dim, q_heads, rep;
  int rotate, axes, max_bits, quant;
  int64_t n_bins, total_bits;
  int shw, n_chunks;
};

// q' = scale * R q (R per 64-channel block) or scale * q; one thread per
// channel (blockDim.x == head_dim), LDS: two head_dim rows.  R = H diag(s) / 8
// with H by the six-stage butterfly network of k_att_final.
__global__ void k_att_qrot(AttArgs a) {
  extern __shared__ float s_q[];
  const int64_t row = static_cast<int64_t>(blockIdx.y) * a.q_heads + blockIdx.x;
  const int i = threadIdx.x;
  float v = a.q[row * a.head_dim + i];
  if (a.rotate) {
    float* x = s_q;
    float* y = s_q + a.head_dim;
    x[i] = v * rotation_sign(i & 63);
    __syncthreads();
#pragma unroll
    for (int bit = 1; bit < 64; bit <<= 1) {
      const float u = x[i], w = x[i ^ bit];
      y[i] = (i & bit) ? w - u : u + w;
      __syncthreads();
      float* t = x;
      x = y;
      y = t;
    }
    v = x[i] * 0.125f;
  }
  a.qrot[row * a.head_dim + i] = a.scale * v;
}

// ---- projections: lane = bin f of kv head h --------------------------------
// The rotated, scaled queries of the kv head are staged in LDS transposed
// (channel-major, the query heads of a channel adjacent), so one broadcast
// read serves every lane.  RQ (a multiple of 4) is at least the number of
// query heads per kv head; the unused heads have zero queries.
template <int WPP, int RQ>
__global__ __launch_bounds__(256) void k_att_proj(AttArgs a) {
  constexpr int D = 64 * WPP;
  __shared__ float s_lv[TACT_CODEBOOK_LEVELS + 1];   // s_lv[0] = 0; b bits at (1 << b) - 1
  __shared__ __attribute__((aligned(16))) float s_qt[D * RQ];   // [channel][r]
  const int h = blockIdx.y;
  const int64_t pair = blockIdx.z;
  for (int j = threadIdx.x; j <= TACT_CODEBOOK_LEVELS; j += blockDim.x)
    s_lv[j] = j ? c_levels_q[a.quant][j - 1] : 0.f;
  const float* qr = a.qrot + (pair * a.q_heads + static_cast<int64_t>(h) * a.rep) * D;
  for (int e = threadIdx.x; e < D * RQ; e += blockDim.x) {
    const int c = e / RQ, r = e % RQ;
    s_qt[e] = r < a.rep ? qr[r * D + c] : 0.f;
  }
  __syncthreads();
  int f = blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = f < a.shw;
  // side info through buffer loads every lane issues (past the buffer: 0)
  const int bin = live ? f * a.kv_heads + h : 0;
  const uint8_t* rk = a.krec.base + pair * a.krec.stride;
  int b = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b8(
      att_rsrc(rk + a.krec.off_bits, a.n_bins), live ? bin : kPastBuffer, 0, 0));
  int64_t p0 = __builtin_amdgcn_raw_buffer_load_b32(
      att_rsrc(a.kpoff + pair * a.n_bins, 4 * a.n_bins), live ? 4 * bin : kPastBuffer, 0, 0);
  float g = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      att_rsrc(rk + a.krec.off_gains, 4 * a.n_bins), live ? 4 * bin : kPastBuffer, 0, 0));
  if (b > a.max_bits || p0 + b > a.total_bits) b = 0;
  float* fld = a.field + (pair * a.q_heads + static_cast<int64_t>(h) * a.rep) * a.shw;
  // A bin without bits projects to 0.  The coded bins of the block are then
  // packed into its first threads (in bin order), so that lanes do not idle
  // on uncoded bins and waves left without a coded bin exit.
  if (live && b == 0)
    for (int r = 0; r < a.rep; ++r) fld[static_cast<int64_t>(r) * a.shw + f] = 0.f;
  __shared__ int s_cnt[256 / kWave];
  __shared__ int4 s_side[256];
  const uint64_t cm = __ballot(b > 0);
  const int wv = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) s_cnt[wv] = static_cast<int>(__popcll(cm));
  __syncthreads();
  int pos = static_cast<int>(__builtin_amdgcn_mbcnt_hi(
      static_cast<uint32_t>(cm >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(cm), 0u)));
  int n = 0;
#pragma unroll
  for (int w = 0; w < 256 / kWave; ++w) {
    if (w < wv) pos += s_cnt[w];
    n += s_cnt[w];
  }
  if (b > 0) s_side[pos] = int4{f, b, static_cast<int>(p0), __float_as_int(g)};
  __syncthreads();
  if (static_cast<int>(threadIdx.x) >= n) return;
  {
    const int4 sd = s_side[threadIdx.x];
    f = sd.x;
    b = sd.y;
    p0 = static_cast<uint32_t>(sd.z);
    g = __int_as_float(sd.w);
  }
  const __amdgpu_buffer_rsrc_t rw = att_rsrc(rk + a.krec.off_codes, a.total_bits * WPP * 8);
  const int base = b > 0 ? (1 << b) - 1 : 0;
  // the largest bit width in the wave bounds the planes read per channel
  int bw = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (__ballot(k < b)) bw = k + 1;
  // query heads in groups of 4 (one 128-bit LDS read per channel and group)
  float acc[RQ];
#pragma unroll
  for (int r = 0; r < RQ; ++r) acc[r] = 0.f;
  // planes decoded per bin: the wave's widest bin rounded up to 1, 2, 4 or 8
  const int nbc = bw <= 1 ? 1 : bw <= 2 ? 2 : bw <= 4 ? 4 : 8;
#pragma unroll
  for (int hw = 0; hw < WPP; ++hw) {
    uint32_t wl[8], wh[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint2 w = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
          rw, k < b ? static_cast<int>(((p0 + k) * WPP + hw) * 8) : kPastBuffer, 0, 0));
      wl[k] = w.x;
      wh[k] = w.y;
    }
    // one code byte per channel: cq[t4] byte i = channel 4 t4 + i
    uint32_t cq[16];
    {
      uint32_t ql[8], qh[8];
      if (nbc == 1) {
        planes_to_codes<1>(wl, ql);
        planes_to_codes<1>(wh, qh);
      } else if (nbc == 2) {
        planes_to_codes<2>(wl, ql);
        planes_to_codes<2>(wh, qh);
      } else if (nbc == 4) {
        planes_to_codes<4>(wl, ql);
        planes_to_codes<4>(wh, qh);
      } else {
        planes_to_codes<8>(wl, ql);
        planes_to_codes<8>(wh, qh);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cq[j] = ql[j];
        cq[8 + j] = qh[j];
      }
    }
#pragma unroll 4
    for (int t4 = 0; t4 < 16; ++t4) {
      const uint32_t codes = cq[t4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jj = 4 * t4 + i;
        const float val = s_lv[base + static_cast<int>((codes >> (8 * i)) & 0xFFu)];
        const float4* qc = reinterpret_cast<const float4*>(s_qt + (64 * hw + jj) * RQ);
#pragma unroll
        for (int r4 = 0; r4 < RQ / 4; ++r4) {
          const float4 qv = qc[r4];
          acc[4 * r4 + 0] = fmaf(val, qv.x, acc[4 * r4 + 0]);
          acc[4 * r4 + 1] = fmaf(val, qv.y, acc[4 * r4 + 1]);
          acc[4 * r4 + 2] = fmaf(val, qv.z, acc[4 * r4 + 2]);
          acc[4 * r4 + 3] = fmaf(val, qv.w, acc[4 * r4 + 3]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RQ; ++r)
    if (r < a.rep) fld[static_cast<int64_t>(r) * a.shw + f] = g * acc[r];
}

// ---- the field of one query head: IDCT3, softmax, DCT3 ---------------------
// One axis of the field in LDS on the matrix cores: the field's lines along
// the axis are the columns of B (16 lines per tile, lane t = line, K rows
// 8g..8g+7 per lane group g), the DCT matrix (or its transpose, inverse) is
// A, split into fp16 hi / lo like the codec's contractions.  Every input x
// of the pass satisfies |x| <= bound < 2^e, so x 2^(14 - e) fits fp16 with
// its lo part; outputs are scaled back.  A wave reads a whole tile before
// writing it, and tiles hold disjoint lines, so the pass runs in place.
// fragment slot of (axis, direction, row tile m, K step, hi / lo, lane)
__device__ __forceinline__ int frag_slot(int axis, int inverse, int m, int ks, int hl, int lane) {
  return ((((axis * 2 + inverse) * 4 + m) * 2 + ks) * 2 + hl) * kWave + lane;
}

// in_mul multiplies the inputs (with the pass's scale, inside the split);
// with MAX the pass returns the largest value it wrote (per thread), else
// -inf.  With gout the outputs go to gout (same indexing) instead of back
// into the field: 16-byte stores of a lane's four consecutive outputs when
// the lines are contiguous and their length a multiple of 4.
template <int NP, bool MAX>
__device__ float mfma_axis_pass(float* fld, int n_lines, int N, int inner, const uint4* frags, int axis,
                                int inverse, int e, float in_mul, float* gout) {
  using F = Frag<NP>;
  using vec = typename F::vec;
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  const int t = lane % 16, g = lane / 16;
  vec ahi[F::MT][F::KSTEPS], alo[F::MT][F::KSTEPS];
#pragma unroll
  for (int m = 0; m < F::MT; ++m)
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks) {
      const uint4 h = frags[frag_slot(axis, inverse, m, ks, 0, lane)];
      const uint4 l = frags[frag_slot(axis, inverse, m, ks, 1, lane)];
      if constexpr (F::KV == 8) {
        ahi[m][ks] = __builtin_bit_cast(vec, h);
        alo[m][ks] = __builtin_bit_cast(vec, l);
      } else {
        ahi[m][ks] = __builtin_bit_cast(vec, uint2{h.x, h.y});
        alo[m][ks] = __builtin_bit_cast(vec, uint2{l.x, l.y});
      }
    }
  const float sc = ldexpf(1.0f, 14 - e) * in_mul;
  const float post = ldexpf(1.0f, e - 26);         // 2^-12 (matrix) / 2^(14 - e)
  float mx = -INFINITY;
  const int n_tiles = (n_lines + 15) / 16;
  const int nw = static_cast<int>(blockDim.x / kWave);
  for (int ti = wv; ti < n_tiles; ti += nw) {
    const int l = 16 * ti + t;
    const bool ok = l < n_lines;
    const int lc = ok ? l : n_lines - 1;
    float* p = fld + (lc / inner) * inner * N + (lc % inner);
    f32x4 acc[F::MT];
#pragma unroll
    for (int m = 0; m < F::MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks) {
      float x[F::KV];
#pragma unroll
      for (int v = 0; v < F::KV; ++v) {
        const int k = ks * F::KPER + F::KV * g + v;
        x[v] = k < N ? p[k * inner] : 0.f;
      }
      uint32_t hw[F::KV / 2], lw[F::KV / 2];
#pragma unroll
      for (int v = 0; v < F::KV; v += 2) {
        hw[v / 2] = split_hi_pair(x[v], sc, x[v + 1], sc);
        lw[v / 2] = split_lo_pair(x[v], sc, x[v + 1], sc, hw[v / 2]);
      }
      const vec bhi = pairs_to_vec<NP>(hw), blo = pairs_to_vec<NP>(lw);
#pragma unroll
      for (int m = 0; m < F::MT; ++m) {
        acc[m] = mfma<NP>(ahi[m][ks], bhi, acc[m]);
        acc[m] = mfma<NP>(alo[m][ks], bhi, acc[m]);
        acc[m] = mfma<NP>(ahi[m][ks], blo, acc[m]);
      }
    }
    if (gout != nullptr) {
      float* q = gout + (p - fld);
      if (inner == 1 && (N & 3) == 0) {
#pragma unroll
        for (int m = 0; m < F::MT; ++m) {
          const int n = 16 * m + 4 * g;
          if (ok && n < N)
            *reinterpret_cast<float4*>(q + n) =
                make_float4(acc[m][0] * post, acc[m][1] * post, acc[m][2] * post, acc[m][3] * post);
        }
      } else {
#pragma unroll
        for (int m = 0; m < F::MT; ++m)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int n = 16 * m + 4 * g + rr;
            if (ok && n < N) q[n * inner] = acc[m][rr] * post;
          }
      }
      continue;
    }
#pragma unroll
    for (int m = 0; m < F::MT; ++m)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int n = 16 * m + 4 * g + rr;
        if (ok && n < N) {
          const float y = acc[m][rr] * post;
          p[n * inner] = y;
          if constexpr (MAX) mx = fmaxf(mx, y);
        }
      }
  }
  return mx;
}

template <bool MAX>
__device__ float axis_pass(float* fld, const AttArgs& a, int axis, int inverse, int e, float in_mul,
                           float* gout = nullptr) {
  // field [S][H][W]; axis 0: lines over (h, w), elements H*W apart; axis 1:
  // lines over (s, w), W apart; axis 2: lines over (s, h), contiguous
  const int N = axis == 0 ? a.S : (axis == 1 ? a.H : a.W);
  const int n_lines = a.shw / N;
  const int inner = axis == 0 ? a.H * a.W : (axis == 1 ? a.W : 1);
  if (N <= 16) return mfma_axis_pass<16, MAX>(fld, n_lines, N, inner, a.frags, axis, inverse, e, in_mul, gout);
  if (N <= 32) return mfma_axis_pass<32, MAX>(fld, n_lines, N, inner, a.frags, axis, inverse, e, in_mul, gout);
  return mfma_axis_pass<64, MAX>(fld, n_lines, N, inner, a.frags, axis, inverse, e, in_mul, gout);
}

// The DCT tables as split fp16 A fragments of the field passes, one block
// per (axis, direction): the axis's matrix (forward) or its transpose
// (inverse), in the lane layout of Frag<NP> for the axis's padded length.
__device__ __forceinline__ uint32_t pack_f16(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}
template <int NP>
__device__ void frags_of(const float* tab, int inverse, uint4* out, int axis) {
  using F = Frag<NP>;
  const int lane = threadIdx.x % kWave;
  if (threadIdx.x >= kWave) return;
  typename F::vec hi[F::MT][F::KSTEPS], lo[F::MT][F::KSTEPS];
  load_afrag<NP>(tab, inverse, lane % 16, lane / 16, hi, lo);
#pragma unroll
  for (int m = 0; m < F::MT; ++m)
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks) {
      uint4 h = uint4{0u, 0u, 0u, 0u}, l = h;
      h.x = pack_f16(hi[m][ks][0], hi[m][ks][1]);
      h.y = pack_f16(hi[m][ks][2], hi[m][ks][3]);
      l.x = pack_f16(lo[m][ks][0], lo[m][ks][1]);
      l.y = pack_f16(lo[m][ks][2], lo[m][ks][3]);
      if constexpr (F::KV == 8) {
        h.z = pack_f16(hi[m][ks][4], hi[m][ks][5]);
        h.w = pack_f16(hi[m][ks][6], hi[m][ks][7]);
        l.z = pack_f16(lo[m][ks][4], lo[m][ks][5]);
        l.w = pack_f16(lo[m][ks][6], lo[m][ks][7]);
      }
      out[frag_slot(axis, inverse, m, ks, 0, lane)] = h;
      out[frag_slot(axis, inverse, m, ks, 1, lane)] = l;
    }
}
__global__ void k_att_frags(AttArgs a) {
  const int axis = blockIdx.x / 2, inverse = blockIdx.x % 2;
  const int N = axis == 0 ? a.S : (axis == 1 ? a.H : a.W);
  const float* tab = a.tab + axis * 4096;
  if (N <= 16) frags_of<16>(tab, inverse, a.frags, axis);
  else if (N <= 32) frags_of<32>(tab, inverse, a.frags, axis);
  else frags_of<64>(tab, inverse, a.frags, axis);
}

__device__ float block_reduce(float v, bool is_max, float* red) {
  // wave reduction, then across the waves of the block through LDS
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float u = __shfl_xor(v, o, kWave);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  v = red[0];
  for (int j = 1; j < static_cast<int>(blockDim.x / kWave); ++j) v = is_max ? fmaxf(v, red[j]) : v + red[j];
  return v;
}

__global__ __launch_bounds__(kFieldThreads) void k_att_field(AttArgs a) {
  extern __shared__ float4 fld_v4[];
  float* fld = reinterpret_cast<float*>(fld_v4);
  __shared__ float red[kFieldThreads / kWave];
  const int64_t row = static_cast<int64_t>(blockIdx.y) * a.q_heads + blockIdx.x;
  float* gf = a.field + row * a.shw;
  // the field into LDS, eight 16-byte loads in flight per thread (a field
  // row starts 16-byte aligned when S*H*W is a multiple of 4)
  float ss = 0.f;
  if ((a.shw & 3) == 0) {
    const int n4 = a.shw / 4;
    const float4* g4 = reinterpret_cast<const float4*>(gf);
    for (int e0 = threadIdx.x; e0 < n4; e0 += 8 * blockDim.x) {
      float4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * blockDim.x;
        x[u] = g4[e < n4 ? e : n4 - 1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * blockDim.x;
        if (e < n4) {
          fld_v4[e] = x[u];
          ss = fmaf(x[u].x, x[u].x, ss);
          ss = fmaf(x[u].y, x[u].y, ss);
          ss = fmaf(x[u].z, x[u].z, ss);
          ss = fmaf(x[u].w, x[u].w, ss);
        }
      }
    }
  } else {
    for (int e = threadIdx.x; e < a.shw; e += blockDim.x) {
      const float x = gf[e];
      fld[e] = x;
      ss = fmaf(x, x, ss);
    }
  }
  // The transforms are orthonormal, so every value of every intermediate
  // field is at most the field's L2 norm: one scale serves all passes.
  ss = block_reduce(ss, false, red);
  int e_in = 0;
  if (ss > 0.f) frexpf(sqrtf(ss) * 1.0001f, &e_in);
  if (!(ss < INFINITY)) e_in = 128;         // the sum overflowed: the largest scale
  // the inverse passes, W then H then S; the last one (the lowest axis
  // transformed) also yields the scores' maximum
  const int last_inv = a.axes ? __builtin_ctz(a.axes) : 3;
  float m = -INFINITY;
  for (int axis = 2; axis > last_inv; --axis)
    if (a.axes & (1 << axis)) {
      axis_pass<false>(fld, a, axis, 1, e_in, 1.0f);
      __syncthreads();
    }
  if (last_inv < 3) {
    m = axis_pass<true>(fld, a, last_inv, 1, e_in, 1.0f);
    __syncthreads();
  } else {
    for (int e = threadIdx.x; e < a.shw; e += blockDim.x) m = fmaxf(m, fld[e]);
  }
  m = block_reduce(m, true, red);
  // p = exp(x - m) / l: each exponential once, as 2^((x - m) log2 e) on
  // v_exp_f32 (the product's rounding, |x - m| 2^-24 in the exponent, costs
  // at most ~1e-6 relative where x - m > -20, below the scores' own error);
  // the division by l is folded into the first forward pass's input scale
  float l = 0.f;
  for (int e = threadIdx.x; e < a.shw; e += blockDim.x) {
    const float v = __builtin_amdgcn_exp2f((fld[e] - m) * 1.44269504088896341f);
    fld[e] = v;
    l += v;
  }
  l = block_reduce(l, false, red);
  const float lse = m + logf(l);
  const float il = 1.0f / l;
  if (a.axes == 0) {
    for (int e = threadIdx.x; e < a.shw; e += blockDim.x) fld[e] *= il;
    __syncthreads();
  }
  // probabilities: L2 norm at most 1; the last forward pass (the highest
  // axis transformed) writes straight to the global field
  const int last_fwd = a.axes ? 31 - __builtin_clz(a.axes) : -1;
  float in_mul = il;
  for (int axis = 0; axis < last_fwd; ++axis)
    if (a.axes & (1 << axis)) {
      axis_pass<false>(fld, a, axis, 0, 1, in_mul);
      in_mul = 1.0f;
      __syncthreads();
    }
  if (last_fwd >= 0)
    axis_pass<false>(fld, a, last_fwd, 0, 1, in_mul, gf);
  else
    for (int e = threadIdx.x; e < a.shw; e += blockDim.x) gf[e] = fld[e];
  if (threadIdx.x == 0) a.lse[row] = lse;
}

// ---- output partial sums: lane = channel, one wave per chunk of bins ------
// Bins are taken 64 at a time.  Lane j loads bin j's side info, its query
// heads' probabilities (folded with the bin's gain) and its plane words, and
// turns the planes into one byte of code per channel (the planes transposed,
// as in the projections), written to LDS.  The wave
// then walks the coded bins: a lane reads its channel's code byte, looks up
// the level and accumulates.  Planes at or past a bin's width were loaded as
// zeros, so the batch is decoded over NB planes (its largest width rounded up
// to 1, 2, 4 or 8) with no branch per bin.  RC is a power of two at least
// the number of query heads per kv head; the unused heads carry probability 0.
template <int WPP, int RC>
struct OutStage {
  // A bin's row: its codes, [word][t4] with byte i = channel 4 t4 + i, then
  // its RC probabilities (at least four dwords, so that the 16-byte writes of
  // consecutive lanes (bins) fall in distinct banks for RC <= 4).
  static constexpr int kCodes = WPP * 16;
  static constexpr int kRow = kCodes + (RC < 4 ? 4 : RC);
  uint32_t code[kWave * kRow];
  float lv[TACT_CODEBOOK_LEVELS + 1];
};

template <int WPP, int RC, int NB>
__device__ __forceinline__ void out_group(OutStage<WPP, RC>& st, const uint32_t (&wk)[8][2 * WPP],
                                          uint64_t todo, int bj, const float (&pg)[RC],
                                          float (&acc)[RC][WPP], int lane) {
  // codes of bin `lane`, one byte per channel (the planes of each 32-channel
  // half transposed)
#pragma unroll
  for (int hw = 0; hw < WPP; ++hw)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t pl[NB], c8[8];
#pragma unroll
      for (int k = 0; k < NB; ++k) pl[k] = wk[k][2 * hw + half];
      planes_to_codes<NB>(pl, c8);
      uint4* dst = reinterpret_cast<uint4*>(st.code + lane * st.kRow + hw * 16 + 8 * half);
      dst[0] = make_uint4(c8[0], c8[1], c8[2], c8[3]);
      dst[1] = make_uint4(c8[4], c8[5], c8[6], c8[7]);
    }
  float* prow = reinterpret_cast<float*>(st.code + lane * st.kRow + st.kCodes);
  if constexpr (RC >= 4) {
#pragma unroll
    for (int r = 0; r < RC; r += 4)
      *reinterpret_cast<float4*>(prow + r) = make_float4(pg[r], pg[r + 1], pg[r + 2], pg[r + 3]);
  } else {
#pragma unroll
    for (int r = 0; r < RC; ++r) prow[r] = pg[r];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // level values of bin j at this lane's channels: the lane reads the dword
  // that holds its channel's code byte (four lanes read the same dword) and
  // extracts the byte
  const uint32_t* cw = st.code + lane / 4;
  const int byte_sh = 8 * (lane % 4);
  auto levels = [&](int j, float (&v)[WPP]) {
    const int b = __builtin_amdgcn_readlane(bj, j);
    const float* lvb = st.lv + ((1 << b) - 1);
#pragma unroll
    for (int hw = 0; hw < WPP; ++hw)
      v[hw] = lvb[__builtin_amdgcn_ubfe(cw[j * st.kRow + hw * 16], byte_sh, 8)];
  };
  // the probabilities of bin j (one broadcast read)
  auto probs = [&](int j, float (&pv)[RC]) {
    const float* pr = reinterpret_cast<const float*>(st.code + j * st.kRow + st.kCodes);
    if constexpr (RC >= 4) {
#pragma unroll
      for (int r = 0; r < RC; r += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(pr + r);
        pv[r] = v4.x;
        pv[r + 1] = v4.y;
        pv[r + 2] = v4.z;
        pv[r + 3] = v4.w;
      }
    } else {
#pragma unroll
      for (int r = 0; r < RC; ++r) pv[r] = pr[r];
    }
  };
  int n = __builtin_popcountll(todo);
  // ST bins per step (independent chains, so the LDS round trips overlap)
  constexpr int ST = (WPP == 4 || RC == 16) ? 2 : 4;
  for (; n >= ST; n -= ST) {
    int j[ST];
    float v[ST][WPP];
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      j[i] = __builtin_ctzll(todo);
      todo &= todo - 1;
    }
    float p[ST][RC];
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      levels(j[i], v[i]);
      probs(j[i], p[i]);
    }
#pragma unroll
    for (int r = 0; r < RC; ++r)
#pragma unroll
      for (int hw = 0; hw < WPP; ++hw)
#pragma unroll
        for (int i = 0; i < ST; ++i) acc[r][hw] = fmaf(p[i][r], v[i][hw], acc[r][hw]);
  }
  for (; n > 0; --n) {
    const int j = __builtin_ctzll(todo);
    todo &= todo - 1;
    float v[WPP], p[RC];
    levels(j, v);
    probs(j, p);
#pragma unroll
    for (int r = 0; r < RC; ++r)
#pragma unroll
      for (int hw = 0; hw < WPP; ++hw) acc[r][hw] = fmaf(p[r], v[hw], acc[r][hw]);
  }
}

template <int WPP, int RC>
__global__ __launch_bounds__(kWave) void k_att_out(AttArgs a) {
  __shared__ OutStage<WPP, RC> st;
  for (int j = threadIdx.x; j <= TACT_CODEBOOK_LEVELS; j += blockDim.x)
    st.lv[j] = j ? c_levels_q[a.quant][j - 1] : 0.f;
  __syncthreads();
  const int lane = threadIdx.x;
  const int chunk = blockIdx.x, h = blockIdx.y;
  const int64_t pair = blockIdx.z;
  const uint8_t* rv = a.vrec.base + pair * a.vrec.stride;
  const __amdgpu_buffer_rsrc_t rw = att_rsrc(rv + a.vrec.off_codes, a.total_bits * WPP * 8);
  const __amdgpu_buffer_rsrc_t rb = att_rsrc(rv + a.vrec.off_bits, a.n_bins);
  const __amdgpu_buffer_rsrc_t rg = att_rsrc(rv + a.vrec.off_gains, 4 * a.n_bins);
  const __amdgpu_buffer_rsrc_t ro = att_rsrc(a.vpoff + pair * a.n_bins, 4 * a.n_bins);
  // the probabilities of this kv head's query heads; heads past a.rep fall
  // past the descriptor's range and read 0
  const __amdgpu_buffer_rsrc_t rp = att_rsrc(
      a.field + (pair * a.q_heads + static_cast<int64_t>(h) * a.rep) * a.shw,
      4 * static_cast<int64_t>(a.rep) * a.shw);
  float acc[RC][WPP];
#pragma unroll
  for (int r = 0; r < RC; ++r)
#pragma unroll
    for (int hw = 0; hw < WPP; ++hw) acc[r][hw] = 0.f;
  const int f_end = min(a.shw, (chunk + 1) * kChunk);
  for (int f0 = chunk * kChunk; f0 < f_end; f0 += kWave) {
    // side info, probabilities and plane words of bins f0 + lane, all
    // through buffer loads that every lane issues (lanes with nothing to
    // read take an offset past the buffer and read 0), so one wait covers
    // each batch
    const int f = f0 + lane;
    const bool ok = f < f_end;
    const int bin = ok ? f * a.kv_heads + h : 0;
    int bj = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b8(rb, ok ? bin : kPastBuffer, 0, 0));
    const int64_t pj = __builtin_amdgcn_raw_buffer_load_b32(ro, ok ? 4 * bin : kPastBuffer, 0, 0);
    const float gj = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rg, ok ? 4 * bin : kPastBuffer, 0, 0));
    float pg[RC];
#pragma unroll
    for (int r = 0; r < RC; ++r)
      pg[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rp, ok && r < a.rep ? 4 * (r * a.shw + f) : kPastBuffer, 0, 0));
    if (bj > a.max_bits || pj + bj > a.total_bits) bj = 0;
#pragma unroll
    for (int r = 0; r < RC; ++r) pg[r] = bj > 0 ? pg[r] * gj : 0.f;
    // plane k of the bin: WPP consecutive 64-bit words
    uint32_t wk[8][2 * WPP];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int off = k < bj ? static_cast<int>((pj + k) * WPP * 8) : kPastBuffer;
      if constexpr (WPP == 1) {
        const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rw, off, 0, 0));
        wk[k][0] = v.x;
        wk[k][1] = v.y;
      } else {
#pragma unroll
        for (int q = 0; q < WPP / 2; ++q) {
          const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 16 * q, 0));
          wk[k][4 * q + 0] = v.x;
          wk[k][4 * q + 1] = v.y;
          wk[k][4 * q + 2] = v.z;
          wk[k][4 * q + 3] = v.w;
        }
      }
    }
    int bw = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (__ballot(k < bj)) bw = k + 1;
    const uint64_t todo = __ballot(bj > 0);
    if (bw <= 1) {
      out_group<WPP, RC, 1>(st, wk, todo, bj, pg, acc, lane);
    } else if (bw <= 2) {
      out_group<WPP, RC, 2>(st, wk, todo, bj, pg, acc, lane);
    } else if (bw <= 4) {
      out_group<WPP, RC, 4>(st, wk, todo, bj, pg, acc, lane);
    } else {
      out_group<WPP, RC, 8>(st, wk, todo, bj, pg, acc, lane);
    }
    // every lane has read the codes before the next group overwrites them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  float* dst = a.partial + ((pair * a.kv_heads + h) * a.n_chunks + chunk) * a.rep * (64 * WPP);
#pragma unroll
  for (int r = 0; r < RC; ++r)
    if (r < a.rep)
#pragma unroll
      for (int hw = 0; hw < WPP; ++hw) dst[r * 64 * WPP + 64 * hw + lane] = acc[r][hw];
}

// ---- sum over chunks, undo the rotation ----------------------------------
// One thread per channel (blockDim.x == head_dim); LDS: two head_dim rows.
// R^T = diag(s) H / 8 on each 64-block: H by a six-stage butterfly network
// (Sylvester order: stage `bit` maps (a, b) at (i, i | bit) to (a + b, a - b)).
__global__ void k_att_final(AttArgs a) {
  extern __shared__ float s_o[];
  const int qh = blockIdx.x;
  const int64_t pair = blockIdx.y;
  const int h = qh / a.rep, r = qh % a.rep;
  const int d = a.head_dim;
  const int i = threadIdx.x;
  const float* src = a.partial + (pair * a.kv_heads + h) * a.n_chunks * a.rep * d + r * d + i;
  const int64_t cs = static_cast<int64_t>(a.rep) * d;       // between chunks
  // four independent partial sums, so the loads are in flight together
  float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
  int c = 0;
  for (; c + 4 <= a.n_chunks; c += 4) {
    v0 += src[c * cs];
    v1 += src[(c + 1) * cs];
    v2 += src[(c + 2) * cs];
    v3 += src[(c + 3) * cs];
  }
  for (; c < a.n_chunks; ++c) v0 += src[c * cs];
  float v = (v0 + v1) + (v2 + v3);
  if (a.rotate) {
    float* x = s_o;
    float* y = s_o + d;
    x[i] = v;
    __syncthreads();
#pragma unroll
    for (int bit = 1; bit < 64; bit <<= 1) {
      const float u = x[i], w = x[i ^ bit];
      y[i] = (i & bit) ? w - u : u + w;
      __syncthreads();
      float* t = x;
      x = y;
      y = t;
    }
    v = x[i] * (0.125f * rotation_sign(i & 63));
  }
  a.out[(pair * a.q_heads + qh) * d + i] = v;
}

}  // namespace

int attend_chunks(const Geometry& g) {
  const int shw = g.S * g.H * g.W;
  return (shw + kChunk - 1) / kChunk;
}

static_assert(kMaxAttendRep == 16, "head capacities below cover 1..16 query heads per kv head");

// the projection kernel for the smallest of 4, 8, 16 that is >= a.rep
template <int WPP>
void launch_proj(dim3 grid, const AttArgs& a, hipStream_t s) {
  if (a.rep <= 4) {
    hipLaunchKernelGGL((k_att_proj<WPP, 4>), grid, dim3(256), 0, s, a);
  } else if (a.rep <= 8) {
    hipLaunchKernelGGL((k_att_proj<WPP, 8>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_att_proj<WPP, 16>), grid, dim3(256), 0, s, a);
  }
}

// the output kernel for the smallest power-of-two head capacity >= a.rep
template <int WPP>
void launch_out(dim3 grid, const AttArgs& a, hipStream_t s) {
  if (a.rep <= 1) {
    hipLaunchKernelGGL((k_att_out<WPP, 1>), grid, dim3(kWave), 0, s, a);
  } else if (a.rep <= 2) {
    hipLaunchKernelGGL((k_att_out<WPP, 2>), grid, dim3(kWave), 0, s, a);
  } else if (a.rep <= 4) {
    hipLaunchKernelGGL((k_att_out<WPP, 4>), grid, dim3(kWave), 0, s, a);
  } else if (a.rep <= 8) {
    hipLaunchKernelGGL((k_att_out<WPP, 8>), grid, dim3(kWave), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_att_out<WPP, 16>), grid, dim3(kWave), 0, s, a);
  }
}

void launch_attend(const Geometry& g, int64_t n_pairs, int q_heads, RecordView krec,
                   RecordView vrec, const uint32_t* kpoff, const uint32_t* vpoff, const float* q,
                   float scale, float* qrot, float* field, float* partial, float* out, float* lse,
                   const float* tab, uint32_t* frags, hipStream_t s) {
  AttArgs a;
  a.krec = krec;
  a.vrec = vrec;
  a.kpoff = kpoff;
  a.vpoff = vpoff;
  a.q = q;
  a.scale = scale;
  a.qrot = qrot;
  a.field = field;
  a.partial = partial;
  a.out = out;
  a.lse = lse;
  a.tab = tab;
  a.frags = reinterpret_cast<uint4*>(frags);
  a.S = g.S;
  a.H = g.H;
  a.W = g.W;
  a.kv_heads = g.kv_heads;
  a.head_dim = g.head_dim;
  a.q_heads = q_heads;
  a.rep = q_heads / g.kv_heads;
  a.rotate = g.rotation == TACT_ROTATION_HADAMARD;
  a.quant = g.quantizer;
  a.axes = g.axes;
  a.max_bits = g.max_bits;
  a.n_bins = g.n_bins;
  a.total_bits = g.total_bits;
  a.shw = g.S * g.H * g.W;
  a.n_chunks = attend_chunks(g);
  const unsigned np = static_cast<unsigned>(n_pairs);
  hipLaunchKernelGGL(k_att_frags, dim3(6), dim3(kWave), 0, s, a);
  hipLaunchKernelGGL(k_att_qrot, dim3(q_heads, np), dim3(g.head_dim),
                     2 * g.head_dim * sizeof(float), s, a);
  const dim3 gp((a.shw + 255) / 256, g.kv_heads, np), go(a.n_chunks, g.kv_heads, np);
  if (g.head_dim == 64) {
    launch_proj<1>(gp, a, s);
  } else if (g.head_dim == 128) {
    launch_proj<2>(gp, a, s);
  } else {
    launch_proj<4>(gp, a, s);
  }
  const size_t lds = static_cast<size_t>(a.shw) * sizeof(float);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_att_field),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  hipLaunchKernelGGL(k_att_field, dim3(q_heads, np), dim3(kFieldThreads), lds, s, a);
  if (g.head_dim == 64) {
    launch_out<1>(go, a, s);
  } else if (g.head_dim == 128) {
    launch_out<2>(go, a, s);
  } else {
    launch_out<4>(go, a, s);
  }
  hipLaunchKernelGGL(k_att_final, dim3(q_heads, np), dim3(g.head_dim),
                     2 * g.head_dim * sizeof(float), s, a);
}

}  // namespace tact
