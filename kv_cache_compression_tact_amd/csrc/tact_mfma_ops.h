// Matrix-core helpers shared by the codec and attention kernels (gfx950):
// fp16 hi/lo splits of fp32 operands, the MFMA fragment layout of one
// contraction, and the DCT matrix fragments.  Include inside namespace
// tact's anonymous namespace, after <type_traits>.
#ifndef TACT_MFMA_OPS_H_
#define TACT_MFMA_OPS_H_

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// scale of the DCT matrix before splitting (keeps C_lo out of fp16
// subnormals); undone on output
constexpr float kMatScale = 4096.0f;

// fp32 -> (hi, lo) fp16 pair with hi = RNE(x), lo = RNE(x - hi); x must be
// below 2^15 in magnitude (callers scale first).  The same hi must serve
// as the operand and in lo's subtraction: an x formed by an inexact product
// is passed through a register barrier first (the compiler would otherwise
// form hi from the fused exact product in one place and from the rounded
// product in the other).
__device__ __forceinline__ void split2(float x, _Float16& hi, _Float16& lo) {
#pragma clang fp contract(off)
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

// The same split for two products a0 * b0 and a1 * b1, packed two halves
// per register: v_fma_mix rounds each product to fp16 (hi), then reads that
// hi back as an fp16 operand and rounds the exactly formed remainder
// a * b - hi to fp16 (lo).  When b is a power of two the product is exact
// and the result equals split2 of the scaled value; otherwise hi + lo
// carries the product to about 22 bits.  Products must stay below 2^15.
// A matrix instruction may read a VGPR only two wait states after a VALU
// write; the compiler's hazard check counts an asm block as one, so each
// block ends with those two itself.
__device__ __forceinline__ uint32_t split_hi_pair(float a0, float b0, float a1, float b1) {
  uint32_t hi;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, 0\n\t"
      "s_nop 1"
      : "=&v"(hi)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
  return hi;
}
__device__ __forceinline__ uint32_t split_lo_pair(float a0, float b0, float a1, float b1, uint32_t hi) {
  uint32_t lo;
  asm("v_fma_mixlo_f16 %0, %1, %2, -%5 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %3, %4, -%5 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(lo)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1), "v"(hi));
  return lo;
}

template <int NP>
struct Frag {
  // K elements per lane per MFMA and number of K steps
  static constexpr int KV = (NP == 16) ? 4 : 8;
  static constexpr int KSTEPS = (NP == 64) ? 2 : 1;
  static constexpr int KPER = (NP == 16) ? 16 : 32;
  static constexpr int MT = NP / 16;
  typedef typename std::conditional<NP == 16, f16x4, f16x8>::type vec;
};

// KV fp16 values from KV / 2 packed pairs
template <int NP>
__device__ __forceinline__ typename Frag<NP>::vec pairs_to_vec(const uint32_t (&w)[Frag<NP>::KV / 2]) {
  if constexpr (Frag<NP>::KV == 8) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(typename Frag<NP>::vec, u4{w[0], w[1], w[2], w[3]});
  } else {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(typename Frag<NP>::vec, u2{w[0], w[1]});
  }
}

template <int NP>
__device__ __forceinline__ f32x4 mfma(typename Frag<NP>::vec a, typename Frag<NP>::vec b, f32x4 c) {
  if constexpr (NP == 16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int NP>
__device__ __forceinline__ void load_afrag(const float* tab, int inverse, int t, int g,
                                           typename Frag<NP>::vec (&ahi)[Frag<NP>::MT][Frag<NP>::KSTEPS],
                                           typename Frag<NP>::vec (&alo)[Frag<NP>::MT][Frag<NP>::KSTEPS]) {
  using F = Frag<NP>;
#pragma unroll
  for (int m = 0; m < F::MT; ++m)
#pragma unroll
    for (int ks = 0; ks < F::KSTEPS; ++ks)
#pragma unroll
      for (int v = 0; v < F::KV; ++v) {
        const int row = 16 * m + t;
        const int col = ks * F::KPER + F::KV * g + v;
        const float c = kMatScale * (inverse ? tab[col * 64 + row] : tab[row * 64 + col]);
        _Float16 h, l;
        split2(c, h, l);
        ahi[m][ks][v] = h;
        alo[m][ks][v] = l;
      }
}

// DCT fragments of one contraction (hi / lo per lane) kept in LDS: built
// once per block, read back right before each contraction
template <int NP>
struct FragLds {
  typename Frag<NP>::vec v[Frag<NP>::MT][Frag<NP>::KSTEPS][2][kWave];
};

template <int NP>
__device__ __forceinline__ void frag_to_lds(FragLds<NP>& f, const float* tab, int inverse, int lane) {
  typename Frag<NP>::vec hi[Frag<NP>::MT][Frag<NP>::KSTEPS], lo[Frag<NP>::MT][Frag<NP>::KSTEPS];
  load_afrag<NP>(tab, inverse, lane % 16, lane / 16, hi, lo);
#pragma unroll
  for (int m = 0; m < Frag<NP>::MT; ++m)
#pragma unroll
    for (int ks = 0; ks < Frag<NP>::KSTEPS; ++ks) {
      f.v[m][ks][0][lane] = hi[m][ks];
      f.v[m][ks][1][lane] = lo[m][ks];
    }
}

// lane offset hidden from the optimizer, so that the fragment reads stay
// next to their contraction instead of being hoisted into registers
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int NP>
__device__ __forceinline__ void frag_from_lds(const FragLds<NP>& f, int lane,
                                              typename Frag<NP>::vec (&hi)[Frag<NP>::MT][Frag<NP>::KSTEPS],
                                              typename Frag<NP>::vec (&lo)[Frag<NP>::MT][Frag<NP>::KSTEPS]) {
  const int l = opaque(lane);
#pragma unroll
  for (int m = 0; m < Frag<NP>::MT; ++m)
#pragma unroll
    for (int ks = 0; ks < Frag<NP>::KSTEPS; ++ks) {
      hi[m][ks] = f.v[m][ks][0][l];
      lo[m][ks] = f.v[m][ks][1][l];
    }
}

#endif  // TACT_MFMA_OPS_H_
