// Mixed-sampling logits processor: temperature, top-k and top-p applied to
// the target's logits before the sampling verifier.
//
// Sources: "EAGLE-2 Speculative Decoding Support for llama.cpp - Phase 1" -
// the speedups are measured under mixed sampling (temperature, top_k,
// top_p); "EAGLE-2: Feature-Level Speculative Decoding Guide", Key
// Architectural Mechanics 3 - a greedy or nucleus-sampling verifier walks the
// tree.
//
// One workgroup of 1024 threads per row.  top-k: a radix select of the k-th
// best selection key (value order bits, then the inverted index: the order
// logit descending, index ascending, with every key distinct), one 8-bit
// digit per pass from the top, with integer histograms in LDS, so the result
// does not depend on thread timing; a pass whose chosen bin holds exactly
// the keys still needed ends the search, and the index digits are examined
// only when tied values straddle the cut.  Each pass streams the row with 16
// loads per thread in flight.  top-p (< 1, with k <= 1024): the k
// kept keys are gathered into LDS, bitonic-sorted, weighted by
// exp((l - l_max) / temperature) in fp64 and summed in rank order to find the
// cut.  A last pass writes the logits with the removed tokens at -inf; each
// thread reads and writes the same elements, so the output may be the input.
#include "common.h"

namespace eagle {

constexpr int kLpThreads = 1024;
constexpr int kLpMaxCand = 1024;
constexpr int kHc = 32;
constexpr int kLpBatch = 16;   // row loads of a thread in flight before the first is used

// Calls f(value, index) for every element of the row this thread owns, with
// the thread's loads for a batch issued before the first is used: 16-byte
// loads (4 consecutive elements, 8 in flight) when the row allows them,
// else single elements (16 in flight).
template <typename F>
__device__ __forceinline__ void for_row(const float* row, int V, int tid, F&& f) {
  if ((V & 3) == 0 && ((uintptr_t)row & 15) == 0) {
    const int V4 = V >> 2;
    const f32x4* r4 = (const f32x4*)row;
    for (int c0 = tid; c0 < V4; c0 += kLpThreads * 8) {
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * kLpThreads;
        x[u] = c < V4 ? r4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * kLpThreads;
        if (c < V4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) f(x[u][e], 4 * c + e);
        }
      }
    }
    return;
  }
  for (int v0 = tid; v0 < V; v0 += kLpThreads * kLpBatch) {
    float x[kLpBatch];
#pragma unroll
    for (int u = 0; u < kLpBatch; ++u) {
      const int v = v0 + u * kLpThreads;
      x[u] = v < V ? row[v] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kLpBatch; ++u) {
      const int v = v0 + u * kLpThreads;
      if (v < V) f(x[u], v);
    }
  }
}

__global__ __launch_bounds__(kLpThreads) void logits_process_kernel(const float* in, int V, int k,
                                                                     double inv_t, float top_p,
                                                                     float* out, int32_t* kept) {
  // kHc copies of the histogram, rows padded to 257 words: lane l adds to
  // copy l mod kHc, so the lanes of one instruction that share a bin hit
  // different copies on different banks (the first digits of nearby logits
  // fall in a handful of bins)
  __shared__ uint32_t hist[kHc][257];
  __shared__ uint32_t htot[256];
  __shared__ selkey_t cand[kLpMaxCand];
  __shared__ double pw[kLpMaxCand];
  __shared__ int sh_bin, sh_rem, sh_exact, ncand, sh_cut;
  __shared__ selkey_t sh_theta;
  const int tid = threadIdx.x;
  const size_t r = blockIdx.x;
  const float* row = in + r * V;
  float* orow = out + r * V;

  // The k-th best key as (th_hi, th_lo): value order bits, inverted index.
  // Kept: ord > th_hi, or ord == th_hi and ~index >= th_lo.  (0, 0) keeps all.
  uint32_t th_hi = 0, th_lo = 0;
  int keep = V;
  if (k < V) {
    const int copy = tid % kHc;
    // one 8-bit digit per pass, value bits first; `word` 1: the value's order
    // bits, 0: the inverted index among the tied values
    auto pass = [&](int word, int sh, uint32_t mask, uint32_t prefix, int rem, int& bin,
                    int& left, bool& exact) __attribute__((always_inline)) {
      for (int i = tid; i < kHc * 257; i += kLpThreads) (&hist[0][0])[i] = 0u;
      __syncthreads();
      if (word) {
        for_row(row, V, tid, [&](float x, int v) {
          const uint32_t o = ord_f32(x);
          if ((o & mask) == prefix) atomicAdd(&hist[copy][(o >> sh) & 255u], 1u);
        });
      } else {
        for_row(row, V, tid, [&](float x, int v) {
          const uint32_t lo = ~(uint32_t)v;
          if (ord_f32(x) == th_hi && (lo & mask) == prefix)
            atomicAdd(&hist[copy][(lo >> sh) & 255u], 1u);
        });
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t c = 0;
#pragma unroll 8
        for (int q = 0; q < kHc; ++q) c += hist[q][tid];
        htot[tid] = c;
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, b = 255;
        for (; b > 0; --b) {
          if (cum + (int)htot[b] >= rem) break;
          cum += (int)htot[b];
        }
        sh_bin = b;
        sh_rem = rem - cum;
        sh_exact = (int)htot[b] == rem - cum;
      }
      __syncthreads();
      bin = sh_bin;
      left = sh_rem;
      exact = sh_exact;
      __syncthreads();  // every thread has read the result before the next reset
    };
    int rem = k;
    bool exact = false;
    uint32_t mask = 0;
    for (int d = 3; d >= 0 && !exact; --d) {
      int bin;
      pass(1, 8 * d, mask, th_hi, rem, bin, rem, exact);
      th_hi |= (uint32_t)bin << (8 * d);
      mask |= 255u << (8 * d);
    }
    // still more values equal to th_hi than tokens left: the lower indices win
    mask = 0;
    for (int d = 3; d >= 0 && !exact; --d) {
      int bin;
      pass(0, 8 * d, mask, th_lo, rem, bin, rem, exact);
      th_lo |= (uint32_t)bin << (8 * d);
      mask |= 255u << (8 * d);
    }
    keep = k;
  }
  auto kept_key = [&](float x, int v) __attribute__((always_inline)) {
    const uint32_t o = ord_f32(x);
    return (o > th_hi) | ((o == th_hi) & (~(uint32_t)v >= th_lo));
  };

  if (top_p < 1.0f) {
    if (tid == 0) ncand = 0;
    __syncthreads();
    for_row(row, V, tid, [&](float x, int v) {
      if (kept_key(x, v)) {
        const int slot = atomicAdd(&ncand, 1);
        if (slot < kLpMaxCand) cand[slot] = sel_key(x, v);
      }
    });
    __syncthreads();
    int N = 1;
    while (N < keep) N <<= 1;
    for (int i = tid; i < N; i += kLpThreads)
      if (i >= keep) cand[i] = 0ull;
    for (int size = 2; size <= N; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        __syncthreads();
        const int i = tid;
        const int j = i ^ stride;
        if (i < N && j > i) {
          const bool desc = (i & size) == 0;
          const selkey_t a = cand[i], b = cand[j];
          if ((a < b) == desc) {
            cand[i] = b;
            cand[j] = a;
          }
        }
      }
    __syncthreads();
    const double l0 = (double)key_value(cand[0]);
    for (int j = tid; j < keep; j += kLpThreads)
      pw[j] = exp(((double)key_value(cand[j]) - l0) * inv_t);
    __syncthreads();
    if (tid == 0) {
      double total = 0.0;
      for (int j = 0; j < keep; ++j) total += pw[j];
      const double target = (double)top_p * total;
      double before = 0.0;
      int c = 0;
      while (c < keep && before < target) {
        before += pw[c];
        ++c;
      }
      sh_cut = c;
      sh_theta = cand[c - 1];
    }
    __syncthreads();
    th_hi = (uint32_t)(sh_theta >> 32);
    th_lo = (uint32_t)sh_theta;
    keep = sh_cut;
  }

  if ((V & 3) == 0 && (((uintptr_t)row | (uintptr_t)orow) & 15) == 0) {
    // 16-byte stores of 4 consecutive outputs (their 4 inputs were read by
    // this same thread in this pass, so the output may be the input)
    const int V4 = V >> 2;
    for (int c0 = tid; c0 < V4; c0 += kLpThreads * 8) {
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * kLpThreads;
        x[u] = c < V4 ? ((const f32x4*)row)[c] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * kLpThreads;
        if (c < V4) {
          f32x4 y;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = kept_key(x[u][e], 4 * c + e) ? x[u][e] : -INFINITY;
          ((f32x4*)orow)[c] = y;
        }
      }
    }
  } else {
    for_row(row, V, tid, [&](float x, int v) { orow[v] = kept_key(x, v) ? x : -INFINITY; });
  }
  if (tid == 0 && kept) kept[r] = keep;
}

}  // namespace eagle

extern "C" int eagle_logits_process(const float* logits, int32_t T, int32_t V, float temperature,
                                    int32_t top_k, float top_p, float* out, int32_t* kept,
                                    hipStream_t stream) {
  using namespace eagle;
  EAGLE_REQUIRE(logits && out, EAGLE_EINVAL);
  EAGLE_REQUIRE(T >= 1 && V >= 1 && top_k >= 0, EAGLE_EINVAL);
  EAGLE_REQUIRE(temperature > 0.0f && temperature < INFINITY, EAGLE_EINVAL);
  EAGLE_REQUIRE(top_p > 0.0f && top_p <= 1.0f, EAGLE_EINVAL);
  const int k = (top_k == 0 || top_k >= V) ? V : top_k;
  EAGLE_REQUIRE(top_p == 1.0f || k <= kLpMaxCand, EAGLE_EUNSUPPORTED);
  hipLaunchKernelGGL(logits_process_kernel, dim3(T), dim3(kLpThreads), 0, stream, logits, V, k,
                     1.0 / (double)temperature, top_p, out, kept);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
