// Device-side helpers shared by the libpa kernels: the pool slab index
// functions (the layout specified in include/pa.h), dtype conversions and the
// E4M3 codec written from the OCP 8-bit floating point format definition.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace pa {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

__host__ __device__ inline bool is_raw_dev(int dt) { return dt == kF32 || dt == kF16 || dt == kBF16; }

// ---- slab index functions (t = token of the block, d = dimension) -------------
// A 32-token block is two 16-token slabs back to back; an 8-token block one
// slab of S = 8.
// raw K: [d/8][t][d%8] within a slab of S tokens
__host__ __device__ inline int raw_k_elem(int t, int d, int BS = 16) {
  const int S = BS == 8 ? 8 : 16, half = t / S;
  return half * 16 * 128 + ((d >> 3) * S + t % S) * 8 + (d & 7);  // halves only with D = 128
}

// raw V: NT = D/16, r = d/NT, T = d%NT, g = t/4, i = t%4
__host__ __device__ inline int raw_v_elem(int t, int d, int D, int BS = 16) {
  const int S = BS == 8 ? 8 : 16, half = t / S, ts = t % S;
  const int nt = D >> 4, r = d / nt, T = d % nt;
  return half * 16 * D + (((T >> 1) * (S >> 2) * 16 + (ts >> 2) * 16 + r) * 2 + (T & 1)) * 4 + (ts & 3);
}

// INT4 K code byte of dimension pair k = d/2
__host__ __device__ inline int int4_k_byte(int t, int k, int D) {
  return (((k & 15) >> 2) * 16 + t) * (D >> 5) * 4 + (k >> 4) * 4 + (k & 3);
}

// INT4 V code byte of dimension pair k = d/2 (d even)
__host__ __device__ inline int int4_v_byte(int t, int k, int D) {
  const int nt = D >> 4, d = 2 * k, r = d / nt, T = d % nt;
  return (((t >> 2) * 16 + r) * (nt >> 1) + (T >> 1)) * 4 + (t & 3);
}

// FP8 K code byte
__host__ __device__ inline int fp8_k_byte(int t, int d) {
  return (((d >> 6) * 4 + ((d & 31) >> 3)) * 16 + t) * 16 + ((d >> 5) & 1) * 8 + (d & 7);
}

// FP8 V code byte
__host__ __device__ inline int fp8_v_byte(int t, int d, int D) {
  const int nt = D >> 4, r = d / nt, T = d % nt;
  return (((T >> 2) * 64 + (t >> 2) * 16 + r) * 4 + (T & 3)) * 4 + (t & 3);
}

// ---- conversions --------------------------------------------------------------
__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ inline uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ inline uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ inline float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ inline float load_as_f32(const void* p, size_t i, int dt) {
  if (dt == kF32) return static_cast<const float*>(p)[i];
  if (dt == kF16) return f16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// ---- E4M3 ("fn": no infinities, 0x7F/0xFF NaN) ------------------------------------
// value = (-1)^s * 2^(e-7) * (1 + m/8) for e > 0, (-1)^s * 2^-6 * m/8 for e = 0
__device__ inline float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  const float mag = e ? ldexpf(float(8 + m), int(e) - 10) : ldexpf(float(m), -9);
  return (c & 0x80) ? -mag : mag;
}

// Nearest E4M3 code to y (finite, |y| <= 448), ties to even, sign of zero kept.
// Every step is exact in fp32 except the final rintf, which rounds to even.
__device__ inline uint32_t e4m3_encode(float y) {
  const uint32_t sign = __float_as_uint(y) >> 31 ? 0x80u : 0u;
  const float a = fabsf(y);
  if (a < 0.015625f) {                    // below 2^-6: subnormal step 2^-9
    return sign | uint32_t(rintf(a * 512.0f));  // 8 becomes the least normal, 0x08
  }
  int ex;
  (void)frexpf(a, &ex);                   // a = f * 2^ex, f in [0.5, 1)
  int E = ex - 1;                         // a in [2^E, 2^(E+1))
  float m = rintf((ldexpf(a, -E) - 1.0f) * 8.0f);
  if (m == 8.0f) {
    E += 1;
    m = 0.0f;
  }
  return sign | (uint32_t(E + 7) << 3) | uint32_t(m);
}

// ---- wave reductions (64 lanes) ------------------------------------------------
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float wave_min(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace pa
