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

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero and touch no memory; the count is clamped to 2^31 - 1 bytes.
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)(bytes < 0x7fffffffull ? bytes : 0x7fffffffull),
                                           kRsrcWord3);
}
// The same for a range that is the same in every lane of the wave: the count
// is made a scalar, so the descriptor lives in SGPRs (a count the compiler
// computes with vector instructions would otherwise make it wrap every load
// in a loop over the distinct descriptors of the wave).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_uniform(const void* base,
                                                                   size_t bytes) {
  const int n = (int)(bytes < 0x7fffffffull ? bytes : 0x7fffffffull);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           __builtin_amdgcn_readfirstlane(n), kRsrcWord3);
}

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt <= lgkm, expcnt
// not waited on.  On gfx9 vmcnt counts vector-memory stores as well as loads.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Hand-off between workgroups without cache-wide write-backs.  Partial tiles
// are written with device-coherent (sc1) buffer stores, which are acknowledged
// only once visible to every XCD, and read with sc1 buffer loads, which never
// hit a stale line in this XCD's L2.  arrive_last first makes every thread
// wait (s_waitcnt vmcnt(0)) until its own stores are acknowledged; only then
// does the barrier let thread 0 count the workgroup's arrival with a
// device-scope atomic.  The workgroup that arrives last of `total` therefore
// finds every other arrival's tile complete, and resets the counter.  Its
// reads are issued after the atomic has returned (thread 0 waits for the
// returned count before the second barrier).  Called by all threads; same
// answer in all.
constexpr int kSc1 = 1 << 4;                     // buffer cache policy bit: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, size_t bytes) {
  return buf_rsrc(base, bytes);
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}

__device__ __forceinline__ bool arrive_last(int32_t* ctr, int total, int* flag) {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));          // own stores acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == total - 1;
    if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}
__device__ __forceinline__ void st_dev2(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kSc1);
}
__device__ __forceinline__ u32x2 ld_dev2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kSc1);
}


__device__ __forceinline__ void set_status(int32_t* st, int32_t bit) {
  if (st) atomicOr(st, bit);
}

// Strict ranking order used by every selection: larger value first, then the
// lower index.  (+0.0 and -0.0 compare equal and fall through to the index.)
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  // bitwise, not short-circuit: compiles to compares and selects, no branches
  return (av > bv) | ((av == bv) & (ai < bi));
}

// ---- selection keys.  The same order as `better` as one unsigned 64-bit
// number: the high word maps the value's bits monotonically (-0.0 folded into
// +0.0, NaN below every number), the low word is the inverted index, so the
// larger key wins and equal values fall to the lower index.  Key 0 is below
// every real (value, index) pair and serves as "none".
typedef unsigned long long selkey_t;

__device__ __forceinline__ uint32_t ord_f32(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u == 0x80000000u) ? 0u : u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (v != v) ? 0u : o;
}
__device__ __forceinline__ selkey_t sel_key(float v, int i) {
  return ((selkey_t)ord_f32(v) << 32) | (uint32_t)(~(uint32_t)i);
}
__device__ __forceinline__ float key_value(selkey_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_index(selkey_t k) { return (int)~(uint32_t)k; }

// ---- cross-lane reductions without the LDS crossbar.
//
// Within a row of 16 lanes the butterfly runs on DPP moves (quad swaps, then
// the half-row and row mirrors); across rows it runs on gfx950's permlane16 /
// permlane32 swaps, which hand both lanes of a pair the two operands in the
// same order.  Every operator used here is commutative, so all 64 lanes end
// with bit-identical results.  All lanes of the wave must be active.
template <int CTRL>
__device__ __forceinline__ int dpp_move(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(dpp_move<CTRL>(__float_as_int(x)));
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppRowMirror = 0x140;   // lane i <-> 15 - i within 16

// (value of the even row, value of the odd row) of the lane's row pair
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(int x, int& a, int& b) {
  const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  a = (int)r[0];
  b = (int)r[1];
}
// (value of lane l % 32, value of lane 32 + l % 32)
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(int x, int& a, int& b) {
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  a = (int)r[0];
  b = (int)r[1];
}

// Combine lanes l, l ^ 16 and l ^ 32 (the four 16-lane rows).
__device__ __forceinline__ float rows_max(float v) {
  float a, b;
  swap16(v, a, b);
  v = fmaxf(a, b);
  swap32(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float rows_sum(float v) {
  float a, b;
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_move<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_move<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_move<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_move<kDppRowMirror>(v));
  return rows_max(v);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<kDppQuadXor1>(v);
  v += dpp_move<kDppQuadXor2>(v);
  v += dpp_move<kDppHalfMirror>(v);
  v += dpp_move<kDppRowMirror>(v);
  return rows_sum(v);
}

__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_move<kDppQuadXor1>(v));
  v = max(v, dpp_move<kDppQuadXor2>(v));
  v = max(v, dpp_move<kDppHalfMirror>(v));
  v = max(v, dpp_move<kDppRowMirror>(v));
  int a, b;
  swap16(v, a, b);
  v = max(a, b);
  swap32(v, a, b);
  return max(a, b);
}

template <int CTRL>
__device__ __forceinline__ double dpp_move(double x) {
  const uint64_t u = __double_as_longlong(x);
  const int lo = dpp_move<CTRL>((int)(uint32_t)u);
  const int hi = dpp_move<CTRL>((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ void swap16(double x, double& a, double& b) {
  const uint64_t u = __double_as_longlong(x);
  int alo, blo, ahi, bhi;
  swap16((int)(uint32_t)u, alo, blo);
  swap16((int)(uint32_t)(u >> 32), ahi, bhi);
  a = __longlong_as_double((long long)(((uint64_t)(uint32_t)ahi << 32) | (uint32_t)alo));
  b = __longlong_as_double((long long)(((uint64_t)(uint32_t)bhi << 32) | (uint32_t)blo));
}
__device__ __forceinline__ void swap32(double x, double& a, double& b) {
  const uint64_t u = __double_as_longlong(x);
  int alo, blo, ahi, bhi;
  swap32((int)(uint32_t)u, alo, blo);
  swap32((int)(uint32_t)(u >> 32), ahi, bhi);
  a = __longlong_as_double((long long)(((uint64_t)(uint32_t)ahi << 32) | (uint32_t)alo));
  b = __longlong_as_double((long long)(((uint64_t)(uint32_t)bhi << 32) | (uint32_t)blo));
}

__device__ __forceinline__ double wave_max_d(double v) {
  v = fmax(v, dpp_move<kDppQuadXor1>(v));
  v = fmax(v, dpp_move<kDppQuadXor2>(v));
  v = fmax(v, dpp_move<kDppHalfMirror>(v));
  v = fmax(v, dpp_move<kDppRowMirror>(v));
  double a, b;
  swap16(v, a, b);
  v = fmax(a, b);
  swap32(v, a, b);
  return fmax(a, b);
}

__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_move<kDppQuadXor1>(v);
  v += dpp_move<kDppQuadXor2>(v);
  v += dpp_move<kDppHalfMirror>(v);
  v += dpp_move<kDppRowMirror>(v);
  double a, b;
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

template <int CTRL>
__device__ __forceinline__ void best_step(float& v, int& i) {
  const float ov = dpp_move<CTRL>(v);
  const int oi = dpp_move<CTRL>(i);
  if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// Best (value, index) pair of lanes l, l ^ 16 and l ^ 32.
__device__ __forceinline__ void rows_best(float& v, int& i) {
  float a, b;
  int ia, ib;
  swap16(v, a, b);
  swap16(i, ia, ib);
  if (better(b, ib, a, ia)) { a = b; ia = ib; }
  swap32(a, v, b);
  swap32(ia, i, ib);
  if (better(b, ib, v, i)) { v = b; i = ib; }
}

template <int CTRL>
__device__ __forceinline__ selkey_t dpp_move(selkey_t x) {
  const int lo = dpp_move<CTRL>((int)(uint32_t)x);
  const int hi = dpp_move<CTRL>((int)(uint32_t)(x >> 32));
  return ((selkey_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ void swap16(selkey_t x, selkey_t& a, selkey_t& b) {
  int alo, blo, ahi, bhi;
  swap16((int)(uint32_t)x, alo, blo);
  swap16((int)(uint32_t)(x >> 32), ahi, bhi);
  a = ((selkey_t)(uint32_t)ahi << 32) | (uint32_t)alo;
  b = ((selkey_t)(uint32_t)bhi << 32) | (uint32_t)blo;
}
__device__ __forceinline__ void swap32(selkey_t x, selkey_t& a, selkey_t& b) {
  int alo, blo, ahi, bhi;
  swap32((int)(uint32_t)x, alo, blo);
  swap32((int)(uint32_t)(x >> 32), ahi, bhi);
  a = ((selkey_t)(uint32_t)ahi << 32) | (uint32_t)alo;
  b = ((selkey_t)(uint32_t)bhi << 32) | (uint32_t)blo;
}
__device__ __forceinline__ selkey_t kmax(selkey_t a, selkey_t b) { return a > b ? a : b; }

// Largest key of lanes l, l ^ 16 and l ^ 32.
__device__ __forceinline__ selkey_t rows_max_key(selkey_t v) {
  selkey_t a, b;
  swap16(v, a, b);
  swap32(kmax(a, b), a, b);
  return kmax(a, b);
}

// Generic butterfly for a commutative operator on float, int, double or selkey_t.
template <typename V, typename Op>
__device__ __forceinline__ V wave_reduce(V v, Op op) {
  v = op(v, dpp_move<kDppQuadXor1>(v));
  v = op(v, dpp_move<kDppQuadXor2>(v));
  v = op(v, dpp_move<kDppHalfMirror>(v));
  v = op(v, dpp_move<kDppRowMirror>(v));
  V a, b;
  swap16(v, a, b);
  v = op(a, b);
  swap32(v, a, b);
  return op(a, b);
}

__device__ __forceinline__ selkey_t wave_max_key(selkey_t v) {
  return wave_reduce(v, [](selkey_t a, selkey_t b) { return kmax(a, b); });
}

// Best (value, index) pair across the wave under `better`.
__device__ __forceinline__ void wave_best(float& v, int& i) {
  best_step<kDppQuadXor1>(v, i);
  best_step<kDppQuadXor2>(v, i);
  best_step<kDppHalfMirror>(v, i);
  best_step<kDppRowMirror>(v, i);
  rows_best(v, i);
}

// Deferred RMSNorm of a product's input rows.  The rows handed over are
// y * gamma (bf16) and row m is to be scaled by 1 / sqrt(mean(y[m]^2) + eps);
// since that scale factors out of the product, consumers apply it to their
// fp32 results.  mean(y^2) arrives as partial sums of squares ssq[p][m]
// (p < parts), added here in p order over n elements.
struct RowNorm {
  const float* ssq;   // [parts][M], or null: no scaling
  int parts;
  int n;
  float eps;
};

// Sum of x[q stride] over q = q0, q0 + step, ... < parts, added in that order.
// The first kPartBatch terms are loaded by strided_load (issued together, so
// that they can stay in flight across other work) and added, with the rest,
// by strided_finish, which loads the rest kPartBatch at a time: a plain loop
// would wait for each load before issuing the next.
constexpr int kPartBatch = 8;
__device__ __forceinline__ void strided_load(const float* x, int parts, size_t stride, int q0,
                                             int step, float (&v)[kPartBatch]) {
#pragma unroll
  for (int u = 0; u < kPartBatch; ++u) {
    const int q = q0 + u * step;
    v[u] = q < parts ? x[(size_t)q * stride] : 0.f;
  }
}
__device__ __forceinline__ float strided_finish(const float* x, int parts, size_t stride, int q0,
                                                int step, const float (&v)[kPartBatch]) {
  float s = 0.f;   // (sums of squares: adding +0 for absent terms changes nothing)
#pragma unroll
  for (int u = 0; u < kPartBatch; ++u) s += v[u];
  for (int b = q0 + kPartBatch * step; b < parts; b += kPartBatch * step) {
    float w[kPartBatch];
    strided_load(x, parts, stride, b, step, w);
#pragma unroll
    for (int u = 0; u < kPartBatch; ++u) s += w[u];
  }
  return s;
}

__device__ __forceinline__ float row_norm_scale(const RowNorm& rn, int M, int m) {
  float v[kPartBatch];
  strided_load(rn.ssq + m, rn.parts, (size_t)M, 0, 1, v);
  const float tot = strided_finish(rn.ssq + m, rn.parts, (size_t)M, 0, 1, v);
  return 1.0f / sqrtf(tot / (float)rn.n + rn.eps);
}

}  // namespace eagle
