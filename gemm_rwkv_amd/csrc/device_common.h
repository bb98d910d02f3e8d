// Device helpers shared by the librq kernels (gfx950, wave64).
//
// Number conversions are written out in integer arithmetic so that their
// rounding does not depend on the hardware's denormal or rounding modes:
// every conversion from fp64 is one round-to-nearest-even step onto the
// target grid, with gradual underflow.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Round the 53-bit significand `sig` (value sig * 2^-52 scaled) right by
// `shift` bits, ties to even.  shift in [1, 63].
__host__ __device__ __forceinline__ uint64_t rne_shift(uint64_t sig, int shift) {
  uint64_t q = sig >> shift;
  uint64_t rem = sig & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  return q;
}

// fp64 -> IEEE binary16, round to nearest even, subnormals kept,
// overflow -> +-inf, NaN -> quiet NaN.
__host__ __device__ __forceinline__ uint16_t f64_to_f16_bits(double v) {
  uint64_t b = __builtin_bit_cast(uint64_t, v);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  uint64_t a = b & 0x7fffffffffffffffull;
  if (a >= 0x7ff0000000000000ull) return sign | (a > 0x7ff0000000000000ull ? 0x7e00u : 0x7c00u);
  int e = (int)(a >> 52);
  if (e == 0) return sign;  // fp64 subnormal: far below half of the fp16 minimum
  int E = e - 1023;
  if (E > 15) return sign | 0x7c00u;
  uint64_t sig = (a & 0x000fffffffffffffull) | 0x0010000000000000ull;
  uint64_t bits;
  if (E >= -14) {
    bits = ((uint64_t)(E + 14) << 10) + rne_shift(sig, 42);
  } else {
    int shift = 28 - E;  // units of 2^-24
    bits = shift > 53 ? 0 : rne_shift(sig, shift);
  }
  if (bits >= 0x7c00u) bits = 0x7c00u;
  return sign | (uint16_t)bits;
}

// fp64 -> IEEE binary32 bits, round to nearest even, subnormals kept.
__host__ __device__ __forceinline__ uint32_t f64_to_f32_bits(double v) {
  uint64_t b = __builtin_bit_cast(uint64_t, v);
  uint32_t sign = (uint32_t)((b >> 32) & 0x80000000u);
  uint64_t a = b & 0x7fffffffffffffffull;
  if (a >= 0x7ff0000000000000ull) return sign | (a > 0x7ff0000000000000ull ? 0x7fc00000u : 0x7f800000u);
  int e = (int)(a >> 52);
  if (e == 0) return sign;
  int E = e - 1023;
  if (E > 127) return sign | 0x7f800000u;
  uint64_t sig = (a & 0x000fffffffffffffull) | 0x0010000000000000ull;
  uint64_t bits;
  if (E >= -126) {
    bits = ((uint64_t)(E + 126) << 23) + rne_shift(sig, 29);
  } else {
    int shift = -E - 97;  // units of 2^-149: sig * 2^(E - 52 + 149)
    bits = shift > 53 ? 0 : rne_shift(sig, shift);
  }
  if (bits >= 0x7f800000u) bits = 0x7f800000u;
  return sign | (uint32_t)bits;
}

// fp64 -> OCP e4m3fn code: nearest value, ties to the even code, magnitudes
// above 448 saturate to 448, sign of zero kept.  Input must be finite.
__host__ __device__ __forceinline__ uint8_t f64_to_e4m3(double v) {
  uint64_t b = __builtin_bit_cast(uint64_t, v);
  uint8_t sign = (uint8_t)((b >> 56) & 0x80u);
  uint64_t a = b & 0x7fffffffffffffffull;
  int e = (int)(a >> 52);
  if (e == 0) return sign;
  int E = e - 1023;
  if (E > 8) return sign | 0x7e;
  uint64_t sig = (a & 0x000fffffffffffffull) | 0x0010000000000000ull;
  uint64_t bits;
  if (E >= -6) {
    bits = ((uint64_t)(E + 6) << 3) + rne_shift(sig, 49);
  } else {
    int shift = 43 - E;  // units of 2^-9
    bits = shift > 53 ? 0 : rne_shift(sig, shift);
  }
  if (bits > 0x7e) bits = 0x7e;
  return sign | (uint8_t)bits;
}

// Exact value of an fp16 bit pattern (finite) as fp64.
__host__ __device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v = e ? ldexp((double)(1024 + m), e - 25) : ldexp((double)m, -24);
  return (h & 0x8000) ? -v : v;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ bool finite_f32(float f) {
  return (__builtin_bit_cast(uint32_t, f) & 0x7f800000u) != 0x7f800000u;
}

// ---- int4 code decoding (weight-streaming products and the int4 GEMM) ----

// packed fp16 pair a - b
__device__ __forceinline__ uint32_t hsub2(uint32_t a, uint32_t b) {
  half2v r = __builtin_bit_cast(half2v, a) - __builtin_bit_cast(half2v, b);
  return __builtin_bit_cast(uint32_t, r);
}

// (v & m) | o in one instruction (v_bitop3_b32, truth table 0xEA)
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t m, uint32_t o) {
  return __builtin_amdgcn_bitop3_b32(v, m, o, 0xEA);
}

// One int4 code word (8 consecutive k: even k in nibbles 0..3 of the low
// half-word, odd k in those of the high half-word) -> fp16 (u - bias) for
// k = 0..7 in natural order.  Nibbles 0 and 2 of both halves land in the
// mantissa of 1024 (ulp 1), nibbles 1 and 3 in that of 64 (ulp 1/16), so each
// pair (2i, 2i + 1) is one AND-OR and one packed subtract of the bias:
// 1032 / 72 for offset-binary symmetric codes (u = q + 8), 1024 / 64 for the
// unsigned superblock codes.
template <bool SIGNED>
__device__ __forceinline__ half8 dec4n(uint32_t v) {
  const uint32_t blo = SIGNED ? 0x64086408u : 0x64006400u;  // 1032 : 1024
  const uint32_t bhi = SIGNED ? 0x54805480u : 0x54005400u;  // 72 : 64
  const uint32_t v8 = v >> 8;
  const uint32_t h0 = hsub2(and_or(v, 0x000f000fu, 0x64006400u), blo);
  const uint32_t h1 = hsub2(and_or(v, 0x00f000f0u, 0x54005400u), bhi);
  const uint32_t h2 = hsub2(and_or(v8, 0x000f000fu, 0x64006400u), blo);
  const uint32_t h3 = hsub2(and_or(v8, 0x00f000f0u, 0x54005400u), bhi);
  return __builtin_bit_cast(half8, make_uint4(h0, h1, h2, h3));
}

// Butterfly reductions over aligned groups of `width` lanes (power of two).
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, width));
  return v;
}

template <int width>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, width));
  return v;
}

template <int width>
__device__ __forceinline__ double group_sum_d(double v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = v + __shfl_xor(v, o, width);
  return v;
}

template <int width>
__device__ __forceinline__ double group_max_d(double v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, width));
  return v;
}

}  // namespace rq
