// Device-side helpers shared by the MLA kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

// ------------------------------------------------------------------ scalar conversions
// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
// two floats -> packed bf16 pair (round to nearest even), low half = a
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// two floats -> packed float16 pair (round to nearest even), low half = a
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // IEEE RNE conversion
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// OCP e4m3 (bias 7, max 448, 0x7f/0xff NaN): decode is exact in float32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xfu;
  uint32_t m = c & 0x7u;
  float v;
  if (e == 0) {
    v = (float)m * 0.001953125f;  // m * 2^-9
  } else {
    v = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));  // 2^(e-7) * (1 + m/8)
  }
  if ((c & 0x7fu) == 0x7fu) v = __builtin_nanf("");
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) | s);
}

// float32 -> e4m3 code: round to nearest even on the exact binary value, saturate at +-448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                      // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;              // >= 448 (incl. inf): saturate
  int e = (int)(a >> 23) - 127;                           // unbiased exponent of |x|
  if (e < -6) {
    // subnormal range of e4m3: value = q * 2^-9 with q in [0, 8]; |x| < 2^-6.
    // q = RNE(|x| * 2^9): exact scaling by a power of two, then integer RNE.
    float s = __builtin_bit_cast(float, a) * 512.0f;     // exact (no underflow: |x| >= 2^-149)
    float q = __builtin_rintf(s);                          // ties to even (default mode)
    return sign | (uint32_t)q;                             // q == 8 gives code 0x08 = 2^-6 (normal)
  }
  // normal: keep 3 mantissa bits, RNE on the 20 dropped bits
  uint32_t mant = a & 0x7fffffu;
  uint32_t keep = mant >> 20;
  uint32_t rest = mant & 0xfffffu;
  uint32_t half = 0x80000u;
  uint32_t eb = (uint32_t)(e + 7);
  uint32_t code = (eb << 3) | keep;
  if (rest > half || (rest == half && (keep & 1u))) code += 1;  // may carry into the exponent
  if (code > 0x7eu) code = 0x7eu;                               // 464 rounds to 448
  return sign | code;
}

// OCP FP6 E2M3 (sign, 2 exponent bits with bias 1, 3 mantissa bits, subnormals m/8, largest
// 7.5, no infinity or NaN): code (low 6 bits) -> value, exact in float32.
__device__ __forceinline__ float e2m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 3u, m = c & 7u;
  const float v = e == 0 ? (float)m * 0.125f : __builtin_bit_cast(float, ((e + 126u) << 23) | (m << 20));
  return (c & 0x20u) ? -v : v;
}

// float32 -> e2m3 code: round to nearest even on the exact binary value, saturate at +-7.5; NaN
// (which the format cannot hold) -> +0.
__device__ __forceinline__ uint32_t f32_to_e2m3(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 26) & 0x20u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0u;                          // NaN
  if (a >= 0x40f00000u) return sign | 0x1fu;              // >= 7.5 (incl. inf): saturate
  const int e = (int)(a >> 23) - 127;                      // a in [2^e, 2^(e+1)), e <= 2
  if (e < 0) {
    // below 1: the grid is k/8, k in [0, 8]; exact scaling by 8, then integer RNE
    const float q = __builtin_rintf(__builtin_bit_cast(float, a) * 8.0f);
    return sign | (uint32_t)q;                             // q == 8 is code 8 = 1.0
  }
  const uint32_t mant = a & 0x7fffffu;
  const uint32_t keep = mant >> 20, rest = mant & 0xfffffu, half = 0x80000u;
  uint32_t code = ((uint32_t)(e + 1) << 3) | keep;
  if (rest > half || (rest == half && (keep & 1u))) code += 1;  // may carry into the exponent
  if (code > 0x1fu) code = 0x1fu;
  return sign | code;
}

// ------------------------------------------------------------------ typed element access
template <int DT> struct Elem;
// ld: load and widen; cvt: widen stored bits (kept raw while a load is in flight, so that the
// conversion does not force a wait at the load)
template <> struct Elem<MLA_F32> {
  typedef float T;
  static __device__ __forceinline__ float cvt(T x) { return x; }
  static __device__ __forceinline__ float ld(const T* p, int64_t i) { return p[i]; }
};
template <> struct Elem<MLA_F16> {
  typedef uint16_t T;
  static __device__ __forceinline__ float cvt(T x) { return f16_bits_to_f32(x); }
  static __device__ __forceinline__ float ld(const T* p, int64_t i) { return f16_bits_to_f32(p[i]); }
};
template <> struct Elem<MLA_BF16> {
  typedef uint16_t T;
  static __device__ __forceinline__ float cvt(T x) { return bf16_bits_to_f32(x); }
  static __device__ __forceinline__ float ld(const T* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
};

// ------------------------------------------------------------------ wave helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Partition of the batch's tokens into G contiguous ranges of (nearly) equal length:
// range p covers global tokens [start(p), start(p+1)) with start(p) = floor(p * total / G).
// Eight float32 values as two bf16 octets whose sum carries ~16 significant bits: hi is the
// round-to-nearest bf16 of each value, lo the bf16 of what hi leaves over (MFMA on both halves
// keeps a float32 operand's precision on the bf16 datapath).
__device__ __forceinline__ void split_hi_lo(const f32x4& v0, const f32x4& v1, bf16x8& bh, bf16x8& bl) {
  uint32_t hv[4], lv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x0 = e < 2 ? v0[2 * e] : v1[2 * e - 4];
    const float x1 = e < 2 ? v0[2 * e + 1] : v1[2 * e - 3];
    const uint32_t h = pack_bf16x2(x0, x1);
    hv[e] = h;
    lv[e] = pack_bf16x2(x0 - __builtin_bit_cast(float, h << 16), x1 - __builtin_bit_cast(float, h & 0xffff0000u));
  }
  bh = __builtin_bit_cast(bf16x8, u32x4{hv[0], hv[1], hv[2], hv[3]});
  bl = __builtin_bit_cast(bf16x8, u32x4{lv[0], lv[1], lv[2], lv[3]});
}

__device__ __forceinline__ int64_t range_start(int64_t p, int64_t total, int64_t G) {
  return (p * total) / G;
}
// Largest p with start(p) <= t, i.e. the range that holds token t.
__device__ __forceinline__ int64_t range_of(int64_t t, int64_t total, int64_t G) {
  return ((t + 1) * G - 1) / total;
}

}  // namespace mla
