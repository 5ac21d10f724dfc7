// Shared device and host helpers for the gfx950 kernels behind eagle.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "eagle.h"

#define EAGLE_LAUNCH_CHECK()                                   \
  do {                                                         \
    if (hipGetLastError() != hipSuccess) return EAGLE_EHIP;    \
  } while (0)

#define EAGLE_REQUIRE(cond, code) \
  do {                            \
    if (!(cond)) return (code);   \
  } while (0)

namespace eagle {

typedef uint16_t bf16_t;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in bits 0-15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return pack_bf16x2(f, 0.0f) & 0xffffu;
}

__device__ __forceinline__ void set_status(int32_t* st, int32_t bit) {
  if (st) atomicOr(st, bit);
}

// Strict ranking order used by every selection: larger value first, then the
// lower index.  (+0.0 and -0.0 compare equal and fall through to the index.)
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Best (value, index) pair across the wave under `better`.
__device__ __forceinline__ void wave_best(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

}  // namespace eagle
