// Device-side helpers shared by the kvcluster kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int D = 128;  // head dimension of the GPU path
constexpr int WAVE = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Element loads of the two supported storage types, widened exactly.
__device__ __forceinline__ float load_f32(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ float load_f32(const float* p, size_t i) { return p[i]; }

// Round an fp64 value once to bf16 (nearest, ties to even), bit pattern out.
// Normal range: add the rounding bias to the fp64 bit pattern and keep its
// top 19 bits (sign, 11 exponent bits, 7 mantissa bits), then rebias the
// exponent from 1023 to 127; a mantissa carry moves into the exponent.
// Below 2^-126 the value is a multiple of 2^-133 after rounding, which rint
// produces from the exactly scaled value.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const unsigned long long mag = u & 0x7FFFFFFFFFFFFFFFull;
  if (mag >= 0x7FF0000000000000ull) return (uint16_t)(sign | (mag > 0x7FF0000000000000ull ? 0x7FC0u : 0x7F80u));
  if (mag < 0x3810000000000000ull) {  // |x| < 2^-126
    const double a = __longlong_as_double((long long)mag) * 0x1p133;
    return (uint16_t)(sign | (uint32_t)rint(a));
  }
  const unsigned long long r = mag + 0x00000FFFFFFFFFFFull + ((mag >> 45) & 1ull);
  const uint32_t e11 = (uint32_t)(r >> 52);
  if (e11 >= 1023u + 128u) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | ((e11 - 896u) << 7) | (uint32_t)((r >> 45) & 0x7Full));
}

// Two adjacent elements (p[0], p[1]) in one load.
__device__ __forceinline__ void load_pair(const uint16_t* p, float& a, float& b) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
  a = __uint_as_float(v << 16);
  b = __uint_as_float(v & 0xFFFF0000u);
}
__device__ __forceinline__ void load_pair(const float* p, float& a, float& b) {
  const float2 v = *reinterpret_cast<const float2*>(p);
  a = v.x;
  b = v.y;
}

// Eight adjacent elements p[0..7] (16-byte aligned) as fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[2 * q] = __uint_as_float(v[q] << 16);
    o[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o[q] = a[q];
    o[4 + q] = b[q];
  }
}

__device__ __forceinline__ void store_op(uint16_t* p, size_t i, double v) { p[i] = f64_to_bf16_rne(v); }
// the value store_op writes, as a double
__device__ __forceinline__ double rounded_op(const uint16_t*, double v) { return (double)bf16_bits_to_f32(f64_to_bf16_rne(v)); }
__device__ __forceinline__ double rounded_op(const float*, double v) { return (double)(float)v; }
__device__ __forceinline__ void store_op(float* p, size_t i, double v) { p[i] = (float)v; }

// Order-preserving map of an fp64 score to uint64 (larger score, larger key);
// -0.0 is folded onto +0.0 first so equal scores give equal keys.
__device__ __forceinline__ unsigned long long ordered_key(double s) {
  s = s + 0.0;
  const unsigned long long u = (unsigned long long)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace kvc
