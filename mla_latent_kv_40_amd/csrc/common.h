// Device-side helpers shared by the libmla kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;       // tokens per cache page
constexpr int kWave = 64;

#define MLA_LDS __attribute__((address_space(3)))

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// The same rounding (nearest even, finite values) in one instruction: v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// ------------------------------------------------------------------ OCP e4m3fn

// Nearest e4m3fn code of x (ties to even), saturating to +-448.  Exact arithmetic only
// (scaling by powers of two and rint), so the result is fully determined by x.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a == a)) return sign | 0x7Fu;          // NaN
  if (a >= 448.0f) return sign | 0x7Eu;        // saturate
  if (a < 0.015625f) {                         // below 2^-6: subnormal multiples of 2^-9
    uint32_t m = (uint32_t)rintf(a * 512.0f);  // 0 .. 8 (8 == smallest normal, code 0x08)
    return sign | m;
  }
  int e;
  float fr = frexpf(a, &e);                    // a = fr * 2^e, fr in [0.5, 1)
  int E = e - 1;                               // a in [2^E, 2^(E+1))
  float q = rintf((fr * 2.0f - 1.0f) * 8.0f);  // mantissa steps of 1/8, nearest even
  int mant = (int)q;
  if (mant == 8) { mant = 0; E += 1; }
  uint32_t code = (uint32_t)((E + 7) << 3) | (uint32_t)mant;
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t E = (c >> 3) & 0xFu, M = c & 7u;
  float v = (E == 0) ? (float)M * (1.0f / 512.0f) : ldexpf(1.0f + (float)M * 0.125f, (int)E - 7);
  return (c & 0x80u) ? -v : v;
}

// ------------------------------------------------------------------ loads

template <typename T>
__device__ __forceinline__ float load_act(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_act<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

// ------------------------------------------------------------------ reductions

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
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// RoPE angle for pair j at position pos, in fp64: pos * base^(-2j/d).
__device__ __forceinline__ void rope_cos_sin(int pos, int j, int d, double base, float* c, float* s) {
  double theta = pow(base, -2.0 * (double)j / (double)d);
  double ang = (double)pos * theta;
  double sn, cs;
  sincos(ang, &sn, &cs);
  *c = (float)cs;
  *s = (float)sn;
}

// Rotated pair in fp64 (cos/sin and products in double), for write-once paths.
__device__ __forceinline__ void rope_pair_f64(float x0, float x1, int pos, int j, int d, double base,
                                              double* y0, double* y1) {
  double theta = pow(base, -2.0 * (double)j / (double)d);
  double ang = (double)pos * theta;
  double sn, cs;
  sincos(ang, &sn, &cs);
  *y0 = (double)x0 * cs - (double)x1 * sn;
  *y1 = (double)x0 * sn + (double)x1 * cs;
}

// fp64 -> bf16 bits with a single rounding (nearest even): round the double directly.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double d) {
  // Split into the float nearest toward zero plus a residual; rounding the float with the
  // sign of the residual as sticky information gives the correctly rounded bf16.
  float f = (float)d;                       // nearest float (may be a double-rounding hazard)
  double r = d - (double)f;
  uint32_t u = __float_as_uint(f);
  uint32_t low = u & 0xFFFFu;
  uint32_t hi = u >> 16;
  // exact halfway in float but not in double: decide by the residual
  if (low == 0x8000u) {
    bool away = (r > 0) == ((u >> 31) == 0);   // residual pushes magnitude up
    if (r == 0) { if (hi & 1u) hi += 1; }
    else if (away) hi += 1;
    return hi & 0xFFFFu;
  }
  if (low > 0x8000u) hi += 1;
  return hi & 0xFFFFu;
}

}  // namespace mla
