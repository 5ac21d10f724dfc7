// Mixed-sampling logits processor: temperature, top-k and top-p applied to
// the target's logits before the sampling verifier.
//
// Sources: "EAGLE-2 Speculative Decoding Support for llama.cpp - Phase 1" -
// the speedups are measured under mixed sampling (temperature, top_k,
// top_p); "EAGLE-2: Feature-Level Speculative Decoding Guide", Key
// Architectural Mechanics 3 - a greedy or nucleus-sampling verifier walks the
// tree.
//
// Two launch shapes.  Rows are cut into chunks of 16384 tokens; when the
// candidates of a row (chunks x k) fit one workgroup (<= 4096 keys),
// lp_chunk_kernel runs one 512-thread workgroup per chunk (32 tokens a
// thread):
// - a lower bound tau of the chunk's k-th value comes from the minimum of
//   group maxima; the elements >= tau (a few percent of a chunk for small k)
//   are staged in LDS and radix-selected there;
// - the chunk's top-k (the row's candidates: every token of the row's top-k
//   is in its chunk's top-k) hand their selection keys to the workspace with
//   device-coherent stores; every other token of the chunk is written -inf;
// - the row's last workgroup to arrive (a self-resetting counter) reads the
//   candidates, radix-selects the row's k-th key, with top-p sorts the k
//   kept and cuts them, and writes each candidate as read or -inf.
// So the row is read from memory about once and written once, and no output
// element is written by two workgroups.  Otherwise (large k) one workgroup
// of 1024 threads per row streams the row once per radix pass.
//
// Selection: a radix select of the k-th best selection key (value order bits,
// then the inverted index: the order logit descending, index ascending, with
// every key distinct), one digit per pass from the top, with integer
// histograms in LDS, so the result does not depend on thread timing; a pass
// whose chosen bin holds exactly the keys still needed ends the search, and
// the index digits are examined only when tied values straddle the cut.  The
// chunk and merge kernels take 11-bit digits starting below the bits that
// every element taking part shares; the row kernel takes 8-bit digits over
// 32 histogram copies.  top-p (< 1, with k <= 1024): the k kept keys in rank
// order are weighted by exp((l - l_max) / temperature) in fp64 and summed in
// rank order to find the cut.  Every output element is written once, by the
// thread that read its input (a candidate: the last workgroup's thread that
// reads it from the input), so the output may be the input.
#include "common.h"

namespace eagle {

constexpr int kLpThreads = 1024;
constexpr int kLpMaxCand = 1024;
constexpr int kHc = 32;
constexpr int kLpBatch = 16;   // row loads of a thread in flight before the first is used
constexpr int kLcThreads = 512;
constexpr int kLcPer = 32;                       // chunk elements held by a thread
constexpr int kLcChunk = kLcThreads * kLcPer;    // 16384 tokens per chunk
constexpr int kLcMaxCand = 4096;                 // chunks x k sorted by one workgroup
constexpr int kLmPer = kLcMaxCand / kLcThreads;   // candidate keys per thread in the merge
constexpr int kLcList = 4096;                    // presented elements staged in LDS

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

// LDS of the radix select.  kHc copies of the histogram, rows padded to 257
// words: lane l adds to copy l mod kHc, so the lanes of one instruction that
// share a bin hit different copies on different banks (the first digits of
// nearby logits fall in a handful of bins).  The copies are zero between
// passes: radix_clear before the first, and each pass clears what it reads.
struct RadixLds {
  uint32_t hist[kHc][257];
  uint32_t htot[256];
  int bin, rem, exact;
};

// Zeroes the histogram copies; a barrier must follow before the first pass.
template <int NT>
__device__ __forceinline__ void radix_clear(RadixLds& s, int tid) {
  for (int i = tid; i < kHc * 257; i += NT) (&s.hist[0][0])[i] = 0u;
}

// The k-th best selection key (k <= the number of elements) among the
// elements that each(f) presents to f(value, index) in this thread, as
// (th_hi, th_lo): value order bits, inverted index.  Kept: ord > th_hi, or
// ord == th_hi and ~index >= th_lo.  [lo, hi] bounds the order bits of every
// presented element, so the digits the two share are fixed without a pass.
// NT threads (>= 256) take part; the histogram copies must be zero (and a
// barrier passed) on entry, and are zero again on return.
template <int NT, typename Each>
__device__ __forceinline__ void radix_select_kth(RadixLds& s, int tid, int k, uint32_t lo,
                                                 uint32_t hi, Each&& each, uint32_t& th_hi,
                                                 uint32_t& th_lo) {
  th_hi = 0;
  th_lo = 0;
  const int copy = tid % kHc;
  // one 8-bit digit per pass, value bits first; `word` 1: the value's order
  // bits, 0: the inverted index among the tied values
  auto pass = [&](int word, int sh, uint32_t mask, uint32_t prefix, int rem, int& bin, int& left,
                  bool& exact) __attribute__((always_inline)) {
    if (word) {
      each([&](float x, int v) {
        const uint32_t o = ord_f32(x);
        if ((o & mask) == prefix) atomicAdd(&s.hist[copy][(o >> sh) & 255u], 1u);
      });
    } else {
      each([&](float x, int v) {
        const uint32_t lo = ~(uint32_t)v;
        if (ord_f32(x) == th_hi && (lo & mask) == prefix)
          atomicAdd(&s.hist[copy][(lo >> sh) & 255u], 1u);
      });
    }
    __syncthreads();
    if (tid < 256) {   // bin tid over the copies, cleared for the next pass
      uint32_t c = 0;
#pragma unroll 8
      for (int q = 0; q < kHc; ++q) {
        c += s.hist[q][tid];
        s.hist[q][tid] = 0u;
      }
      s.htot[tid] = c;
    }
    __syncthreads();
    if (tid < 64) {
      // wave 0: lane L holds bins 4L..4L+3, a suffix scan across the lanes
      // gives the count above each bin, and the bin where the count from the
      // top first reaches rem is published by its lane
      const uint4 c4 = *(const uint4*)&s.htot[4 * tid];
      const uint32_t c[4] = {c4.x, c4.y, c4.z, c4.w};
      const uint32_t own = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = own;   // bins 4 * tid and above
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(incl, off, 64);
        if (tid + off < 64) incl += y;
      }
      int cum = (int)(incl - own);   // bins above 4 * tid + 3
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (cum < rem && cum + (int)c[e] >= rem) {
          s.bin = 4 * tid + e;
          s.rem = rem - cum;
          s.exact = (int)c[e] == rem - cum;
        }
        cum += (int)c[e];
      }
    }
    __syncthreads();
    bin = s.bin;
    left = s.rem;
    exact = s.exact;
    // the next pass publishes again only after two more barriers
  };
  int rem = k;
  bool exact = false;
  uint32_t mask = 0;
  int d = 3;
  const uint32_t diff = lo ^ hi;
  for (; d >= 0 && ((diff >> (8 * d)) & 255u) == 0u; --d) {   // digits every element shares
    th_hi |= hi & (255u << (8 * d));
    mask |= 255u << (8 * d);
  }
  for (; d >= 0 && !exact; --d) {
    int bin;
    pass(1, 8 * d, mask, th_hi, rem, bin, rem, exact);
    th_hi |= (uint32_t)bin << (8 * d);
    mask |= 255u << (8 * d);
  }
  // still more values equal to th_hi than tokens left: the lower indices win
  mask = 0;
  for (d = 3; d >= 0 && !exact; --d) {
    int bin;
    pass(0, 8 * d, mask, th_lo, rem, bin, rem, exact);
    th_lo |= (uint32_t)bin << (8 * d);
    mask |= 255u << (8 * d);
  }
}

// ---- lean radix select, for a few thousand presented elements at most per
// workgroup: one histogram of up to 2048 bins (no copies), padded one word per
// 32 bins so that wave 0's reads of 32 consecutive bins per lane do not
// collide.  Digits of up to 11 bits start just below the bits that every
// presented element shares, so one or two passes usually settle the value.
constexpr int kLnBits = 11;
constexpr int kLnBins = 1 << kLnBits;

struct LeanLds {
  uint32_t hist[kLnBins + kLnBins / 32];
  int bin, rem, exact;
};

__device__ __forceinline__ int lean_slot(uint32_t b) { return (int)(b + (b >> 5)); }

// Zeroes the histogram; a barrier must follow before the first pass.
template <int NT>
__device__ __forceinline__ void lean_clear(LeanLds& s, int tid) {
  for (int i = tid; i < kLnBins + kLnBins / 32; i += NT) s.hist[i] = 0u;
}

// One digit of the k-th best key over one 32-bit word.  `word` 1: the value's
// order bits, [lo, hi] bounding those of every presented element; 0: the
// inverted index among the elements whose order bits equal th_hi, [lo, hi]
// bounding the inverted indices.  Returns the word's bits in `th` and
// whether the last pass's bin held exactly the elements still needed.
template <int NT, typename Each>
__device__ __forceinline__ void lean_word(LeanLds& s, int tid, int word, uint32_t th_hi,
                                          uint32_t lo, uint32_t hi, int& rem, bool& exact,
                                          Each&& each, uint32_t& th) {
  const uint32_t diff = lo ^ hi;
  if (diff == 0u) {   // every presented element has these bits
    th = hi;
    return;
  }
  int hb = 31 - __clz(diff);
  uint32_t mask = hb == 31 ? 0u : ~((2u << hb) - 1u);
  th = hi & mask;
  while (hb >= 0 && !exact) {
    const int w = min(kLnBits, hb + 1);
    const int sh = hb - w + 1;
    const uint32_t dm = (1u << w) - 1u;
    const uint32_t prefix = th;
    each([&](float x, int v) {
      const uint32_t o = ord_f32(x);
      const uint32_t u = word ? o : ~(uint32_t)v;
      if ((word || o == th_hi) && (u & mask) == prefix)
        atomicAdd(&s.hist[lean_slot((u >> sh) & dm)], 1u);
    });
    __syncthreads();
    if (tid < 64) {
      // lane L: bins [32 L, 32 L + 32) (those past the digit's range are
      // zero), read together; a suffix scan across the lanes gives the count
      // above each lane's bins, the lane holding the bin where the count from
      // the top reaches rem publishes it, and every bin is cleared for the
      // next pass
      const int s0 = lean_slot(32u * tid);
      // 8 reads in flight per step, a few registers
      uint32_t own = 0u;
#pragma unroll 1
      for (int i0 = 0; i0 < 32; i0 += 8) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = s.hist[s0 + i0 + i];
#pragma unroll
        for (int i = 0; i < 8; ++i) own += h[i];
      }
      uint32_t incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(incl, off, 64);
        if (tid + off < 64) incl += y;
      }
      int cum = (int)(incl - own);
#pragma unroll 1
      for (int i0 = 24; i0 >= 0; i0 -= 8) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = s.hist[s0 + i0 + i];
#pragma unroll
        for (int i = 7; i >= 0; --i) {
          const int c = (int)h[i];
          if (cum < rem && cum + c >= rem) {
            s.bin = 32 * tid + i0 + i;
            s.rem = rem - cum;
            s.exact = c == rem - cum;
          }
          cum += c;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) s.hist[s0 + i0 + i] = 0u;
      }
    }
    __syncthreads();
    th |= (uint32_t)s.bin << sh;
    rem = s.rem;
    exact = s.exact;
    mask |= dm << sh;
    hb = sh - 1;
    // the next pass publishes again only after its first barrier
  }
}

// The k-th best selection key among the presented elements as (th_hi,
// th_lo), as radix_select_kth; [lo, hi] bounds their order bits and
// [ilo, ihi] their inverted indices.  The histogram must be zero (and a
// barrier passed) on entry, and is zero again on return.
template <int NT, typename Each>
__device__ __forceinline__ void radix_select_lean(LeanLds& s, int tid, int k, uint32_t lo,
                                                  uint32_t hi, uint32_t ilo, uint32_t ihi,
                                                  Each&& each, uint32_t& th_hi, uint32_t& th_lo) {
  int rem = k;
  bool exact = false;
  lean_word<NT>(s, tid, 1, 0u, lo, hi, rem, exact, each, th_hi);
  th_lo = 0u;
  if (!exact) lean_word<NT>(s, tid, 0, th_hi, ilo, ihi, rem, exact, each, th_lo);
}

__device__ __forceinline__ bool kept_key(float x, int v, uint32_t th_hi, uint32_t th_lo) {
  const uint32_t o = ord_f32(x);
  return (o > th_hi) | ((o == th_hi) & (~(uint32_t)v >= th_lo));
}

// Descending bitonic sort of s[0, N) (N a power of two) by NT threads.
template <int NT>
__device__ __forceinline__ void bitonic_desc(selkey_t* s, int N, int tid) {
  for (int size = 2; size <= N; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int p = tid; p < (N >> 1); p += NT) {
        const int i = 2 * p - (p & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const selkey_t a = s[i], b = s[j];
        if ((a < b) == desc) {
          s[i] = b;
          s[j] = a;
        }
      }
    }
  __syncthreads();
}

// Top-p over the first `keep` keys of s (sorted descending): the shortest
// prefix whose fp64 weight sum, in rank order, reaches top_p times the total.
// Returns the prefix length; pw holds >= keep doubles.
template <int NT>
__device__ __forceinline__ int top_p_cut(const selkey_t* s, int keep, double inv_t, float top_p,
                                         double* pw, int* sh_cut, int tid) {
  const double l0 = (double)key_value(s[0]);
  for (int j = tid; j < keep; j += NT) pw[j] = exp(((double)key_value(s[j]) - l0) * inv_t);
  __syncthreads();
  if (tid == 0) {
    double total = 0.0;
    for (int j = 0; j < keep; ++j) total += pw[j];
    const double target = (double)top_p * total;
    // tokens whose preceding mass is below the target (the prefix sums are
    // nondecreasing); no early exit, so the reads need not wait on the test
    double before = 0.0;
    int c = 0;
    for (int j = 0; j < keep; ++j) {
      c += before < target;
      before += pw[j];
    }
    *sh_cut = c;
  }
  __syncthreads();
  return *sh_cut;
}

// One workgroup per row: the row is streamed once per radix pass.
__global__ __launch_bounds__(kLpThreads) void logits_process_kernel(const float* in, int V, int k,
                                                                     double inv_t, float top_p,
                                                                     float* out, int32_t* kept) {
  __shared__ RadixLds rl;
  __shared__ selkey_t cand[kLpMaxCand];
  __shared__ double pw[kLpMaxCand];
  __shared__ int ncand, sh_cut;
  const int tid = threadIdx.x;
  const size_t r = blockIdx.x;
  const float* row = in + r * V;
  float* orow = out + r * V;

  uint32_t th_hi = 0, th_lo = 0;
  int keep = V;
  if (k < V) {
    radix_clear<kLpThreads>(rl, tid);
    __syncthreads();
    radix_select_kth<kLpThreads>(
        rl, tid, k, 0u, 0xffffffffu,
        [&](auto&& f) __attribute__((always_inline)) { for_row(row, V, tid, f); }, th_hi, th_lo);
    keep = k;
  }

  if (top_p < 1.0f) {
    if (tid == 0) ncand = 0;
    __syncthreads();
    for_row(row, V, tid, [&](float x, int v) {
      if (kept_key(x, v, th_hi, th_lo)) {
        const int slot = atomicAdd(&ncand, 1);
        if (slot < kLpMaxCand) cand[slot] = sel_key(x, v);
      }
    });
    __syncthreads();
    int N = 1;
    while (N < keep) N <<= 1;
    for (int i = tid; i < N; i += kLpThreads)
      if (i >= keep) cand[i] = 0ull;
    bitonic_desc<kLpThreads>(cand, N, tid);
    keep = top_p_cut<kLpThreads>(cand, keep, inv_t, top_p, pw, &sh_cut, tid);
    th_hi = (uint32_t)(cand[keep - 1] >> 32);
    th_lo = (uint32_t)cand[keep - 1];
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
          for (int e = 0; e < 4; ++e)
            y[e] = kept_key(x[u][e], 4 * c + e, th_hi, th_lo) ? x[u][e] : -INFINITY;
          ((f32x4*)orow)[c] = y;
        }
      }
    }
  } else {
    for_row(row, V, tid,
            [&](float x, int v) { orow[v] = kept_key(x, v, th_hi, th_lo) ? x : -INFINITY; });
  }
  if (tid == 0 && kept) kept[r] = keep;
}

// Chunk c of row t (grid T x chunks: rows in x, up to 2^31 - 1 of them):
// tokens [c * kLcChunk, +n).  VEC: the
// thread's elements are 8 groups of 4 consecutive tokens, group u at
// 4 * (u * kLcThreads + tid); else 32 single tokens at j * kLcThreads + tid.
// Writes -inf over the chunk's tokens outside its top-min(k, n), and the keys
// of its top-min(k, n) to cand[(t * chunks + c) * k, +min(k, n)) in no
// particular order; the row's last workgroup to arrive at ctr[t] then merges
// the row (and resets ctr[t]).
template <bool VEC>
__global__ __launch_bounds__(kLcThreads, 4) void lp_chunk_kernel(const float* in, int V, int k,
                                                                 double inv_t, float top_p,
                                                                 float* out, int32_t* kept,
                                                                 selkey_t* cand, int32_t* ctr) {
  __shared__ LeanLds rl;
  __shared__ int sh_n, sh_m, sh_flag, sh_cut;
  __shared__ float sh_lo[kLcThreads / 64], sh_hi[kLcThreads / 64];
  __shared__ __align__(16) float lx[kLcList];   // reused by the merge: keys, then weights
  __shared__ __align__(16) int lv[kLcList];
  const int tid = threadIdx.x;
  const int c = blockIdx.y;
  const size_t t = blockIdx.x;
  const int base = c * kLcChunk;
  const int n = min(kLcChunk, V - base);
  const int kc = min(k, n);
  const float* row = in + t * V;
  float* orow = out + t * V;
  auto index = [&](int j) __attribute__((always_inline)) {
    return VEC ? base + 4 * ((j >> 2) * kLcThreads + tid) + (j & 3) : base + j * kLcThreads + tid;
  };

  // every load is issued, from a clamped address, before any is used (a
  // load under a branch would wait at the join); lanes past the chunk read
  // its last element and ignore it
  float x[kLcPer];
  if (VEC) {
#pragma unroll
    for (int u = 0; u < kLcPer / 4; ++u) {
      const int off = min(4 * (u * kLcThreads + tid), n - 4);   // n is a multiple of 4 here
      const f32x4 y = *(const f32x4*)(row + base + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * u + e] = y[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < kLcPer; ++j) x[j] = row[base + min(j * kLcThreads + tid, n - 1)];
  }
  if (tid == 0) {
    sh_n = 0;
    sh_m = 0;
  }

  uint32_t th_hi = 0, th_lo = 0;
  if (kc < n) {
    // A lower bound tau of the chunk's kc-th value: the lanes form at least
    // P >= kc groups (P a power of two, kc <= 512; a group stays in one
    // wave), and the smallest of the group maxima has at least one element
    // per group (its maximum) at or above it.  A group
    // without elements, or kc > 512, gives tau = -inf.  Only elements >= tau
    // take part in the select, and [ord(tau), ord(chunk max)] bounds them.
    lean_clear<kLcThreads>(rl, tid);
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kLcPer; ++j)
      mx = (index(j) - base < n) & (x[j] > mx) ? x[j] : mx;
    int P = 1;
    while (P < kc) P <<= 1;
    const int g = P <= kLcThreads ? min(kLcThreads / P, 64) : 1;   // lanes per group, in one wave
    float gm = mx;
    for (int o = 1; o < g; o <<= 1) gm = fmaxf(gm, __shfl_xor(gm, o, 64));
    float lo_w = wave_reduce(gm, [](float a, float b) { return fminf(a, b); });
    float hi_w = wave_reduce(mx, [](float a, float b) { return fmaxf(a, b); });
    if ((tid & 63) == 0) {
      sh_lo[tid >> 6] = lo_w;
      sh_hi[tid >> 6] = hi_w;
    }
    __syncthreads();
    float tau = sh_lo[0], cmax = sh_hi[0];
#pragma unroll
    for (int w = 1; w < kLcThreads / 64; ++w) {
      tau = fminf(tau, sh_lo[w]);
      cmax = fmaxf(cmax, sh_hi[w]);
    }
    if (P > kLcThreads) tau = -INFINITY;
    // the elements >= tau go to an LDS list (one slot reservation per
    // thread), so the passes need not keep the chunk's registers busy; a
    // list that overflows (a flat or heavily tied chunk) leaves the passes to
    // re-read the chunk from memory
    uint32_t pm = 0u;
#pragma unroll
    for (int j = 0; j < kLcPer; ++j) pm |= (uint32_t)((index(j) - base < n) & (x[j] >= tau)) << j;
    if (pm) {
      int at = atomicAdd(&sh_m, __popc(pm));
#pragma unroll
      for (int j = 0; j < kLcPer; ++j)
        if ((pm >> j) & 1u) {
          if (at < kLcList) {
            lx[at] = x[j];
            lv[at] = index(j);
          }
          ++at;
        }
    }
    __syncthreads();
    const int m = sh_m;
    const uint32_t lo = ord_f32(tau), hi = ord_f32(cmax);
    const uint32_t ilo = ~(uint32_t)(base + n - 1), ihi = ~(uint32_t)base;
    if (m <= kLcList) {
      radix_select_lean<kLcThreads>(
          rl, tid, kc, lo, hi, ilo, ihi,
          [&](auto&& f) __attribute__((always_inline)) {
            for (int i = tid; i < m; i += kLcThreads) f(lx[i], lv[i]);
          },
          th_hi, th_lo);
    } else {
      radix_select_lean<kLcThreads>(
          rl, tid, kc, lo, hi, ilo, ihi,
          [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll 1
            for (int j0 = 0; j0 < kLcPer; j0 += 8) {   // 8 loads in flight
              float y[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) y[j] = row[min(index(j0 + j), base + n - 1)];
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int v = index(j0 + j);
                if ((v - base < n) & (y[j] >= tau)) f(y[j], v);
              }
            }
          },
          th_hi, th_lo);
    }
  }
  __syncthreads();   // sh_n is cleared

  // one slot reservation per thread for its kept elements (few threads
  // have any), then the keys in element order from that slot, stored
  // device-coherently for the row's last workgroup
  const int chunks = gridDim.y;
  const __amdgpu_buffer_rsrc_t rc =
      dev_rsrc(cand + t * chunks * (size_t)k, (size_t)chunks * k * sizeof(selkey_t));
  uint32_t km = 0u;   // kept-element bits
#pragma unroll
  for (int j = 0; j < kLcPer; ++j) {
    const int v = index(j);
    km |= (uint32_t)((v - base < n) & kept_key(x[j], v, th_hi, th_lo)) << j;
  }
  if (km) {
    int slot = atomicAdd(&sh_n, __popc(km));
#pragma unroll
    for (int j = 0; j < kLcPer; ++j)
      if ((km >> j) & 1u) {
        if (slot < kc) {
          const selkey_t key = sel_key(x[j], index(j));
          st_dev2(rc, (uint32_t)((c * k + slot) * sizeof(selkey_t)),
                  u32x2{(uint32_t)key, (uint32_t)(key >> 32)});
        }
        ++slot;
      }
  }
  // The chunk's output: -inf for every token outside its top-k.  Its top-k
  // (the row's candidates) are left to the row's last workgroup, which writes
  // each as read or -inf, so no output element is written by two workgroups.
  if (VEC) {
#pragma unroll
    for (int u = 0; u < kLcPer / 4; ++u) {
      const int off = 4 * (u * kLcThreads + tid);
      if (off < n) {
        const uint32_t q = (km >> (4 * u)) & 15u;
        if (q == 0u) {
          *(f32x4*)(orow + base + off) = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (!((q >> e) & 1u)) orow[base + off + e] = -INFINITY;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kLcPer; ++j) {
      const int off = j * kLcThreads + tid;
      if (off < n && !((km >> j) & 1u)) orow[base + off] = -INFINITY;
    }
  }
  if (!arrive_last(ctr + t, chunks, &sh_flag)) return;

  // ---- the row's last workgroup: the merge.  The candidates (<= kLcMaxCand
  // keys, every token of the row's top-k among them) are radix-selected for
  // the row's k-th key in registers; with top-p the k kept keys are sorted
  // in LDS (over the staging list) and cut.
  lean_clear<kLcThreads>(rl, tid);
  const int kf = min(k, kLcChunk);                                   // full chunks
  const int kl = min(k, V - (chunks - 1) * kLcChunk);               // the last chunk
  const int M = (chunks - 1) * kf + kl;
  selkey_t key[kLmPer];
#pragma unroll
  for (int j = 0; j < kLmPer; ++j) {
    const int i = min(j * kLcThreads + tid, M - 1);
    const int cc = min(i / kf, chunks - 1);
    const u32x2 w = ld_dev2(rc, (uint32_t)((cc * k + (i - cc * kf)) * sizeof(selkey_t)));
    key[j] = j * kLcThreads + tid < M ? (((selkey_t)w.y << 32) | w.x) : 0ull;
  }
  if (tid == 0) sh_n = 0;
  uint32_t mh = 0u, ml = 0u;
  if (k < M) {
    // [lo, hi]: the order bits of the smallest and largest candidate
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int j = 0; j < kLmPer; ++j)
      if (key[j] != 0ull) {
        lo = min(lo, (uint32_t)(key[j] >> 32));
        hi = max(hi, (uint32_t)(key[j] >> 32));
      }
    lo = (uint32_t)wave_reduce((int)lo, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
    hi = (uint32_t)wave_reduce((int)hi, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
    if ((tid & 63) == 0) {
      ((uint32_t*)sh_lo)[tid >> 6] = lo;
      ((uint32_t*)sh_hi)[tid >> 6] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kLcThreads / 64; ++w) {
      lo = min(lo, ((uint32_t*)sh_lo)[w]);
      hi = max(hi, ((uint32_t*)sh_hi)[w]);
    }
    radix_select_lean<kLcThreads>(
        rl, tid, k, lo, hi, ~(uint32_t)(V - 1), 0xffffffffu,
        [&](auto&& f) __attribute__((always_inline)) {
#pragma unroll
          for (int j = 0; j < kLmPer; ++j)
            if (key[j] != 0ull) f(key_value(key[j]), key_index(key[j]));
        },
        mh, ml);
  }
  __syncthreads();   // sh_n is cleared
  const selkey_t th = ((selkey_t)mh << 32) | ml;
  selkey_t cut = th;   // candidates below it become -inf
  int keep = k;
  if (top_p < 1.0f) {
    selkey_t* sk = (selkey_t*)lx;    // the staging list is free now
    double* pw = (double*)lv;
#pragma unroll
    for (int j = 0; j < kLmPer; ++j)
      if (key[j] != 0ull && key[j] >= th) {
        const int slot = atomicAdd(&sh_n, 1);
        if (slot < kLpMaxCand) sk[slot] = key[j];
      }
    __syncthreads();
    int N = 1;
    while (N < k) N <<= 1;
    for (int i = k + tid; i < N; i += kLcThreads) sk[i] = 0ull;
    bitonic_desc<kLcThreads>(sk, N, tid);
    keep = top_p_cut<kLcThreads>(sk, k, inv_t, top_p, pw, &sh_cut, tid);
    cut = sk[keep - 1];
  }
  const float* irow = row;
#pragma unroll
  for (int j = 0; j < kLmPer; ++j)
    if (key[j] != 0ull) {
      const int v = key_index(key[j]);
      if ((unsigned)v < (unsigned)V) orow[v] = key[j] >= cut ? irow[v] : -INFINITY;
    }
  if (tid == 0 && kept) kept[t] = keep;
}

// Chunks of a row, and whether its candidates fit one merge workgroup.
static inline int lp_chunks(int V) { return (V + kLcChunk - 1) / kLcChunk; }
static inline bool lp_chunked(int V, int k) { return (long long)lp_chunks(V) * k <= kLcMaxCand; }
static inline size_t lp_ctr_bytes(int T) { return ((size_t)T * sizeof(int32_t) + 255) / 256 * 256; }

}  // namespace eagle

extern "C" size_t eagle_logits_process_workspace(int32_t T, int32_t V, int32_t top_k) {
  using namespace eagle;
  if (T < 1 || V < 1 || top_k < 0) return 0;
  const int k = (top_k == 0 || top_k >= V) ? V : top_k;
  if (!lp_chunked(V, k)) return 0;
  return lp_ctr_bytes(T) + (size_t)T * lp_chunks(V) * k * sizeof(selkey_t);
}

extern "C" int eagle_logits_process(const float* logits, int32_t T, int32_t V, float temperature,
                                    int32_t top_k, float top_p, float* out, int32_t* kept,
                                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  using namespace eagle;
  EAGLE_REQUIRE(logits && out, EAGLE_EINVAL);
  EAGLE_REQUIRE(T >= 1 && V >= 1 && top_k >= 0, EAGLE_EINVAL);
  EAGLE_REQUIRE(temperature > 0.0f && temperature < INFINITY, EAGLE_EINVAL);
  EAGLE_REQUIRE(top_p > 0.0f && top_p <= 1.0f, EAGLE_EINVAL);
  const int k = (top_k == 0 || top_k >= V) ? V : top_k;
  EAGLE_REQUIRE(top_p == 1.0f || k <= kLpMaxCand, EAGLE_EUNSUPPORTED);
  const double inv_t = 1.0 / (double)temperature;
  const size_t need = eagle_logits_process_workspace(T, V, top_k);
  if (need == 0) {
    hipLaunchKernelGGL(logits_process_kernel, dim3(T), dim3(kLpThreads), 0, stream, logits, V, k,
                       inv_t, top_p, out, kept);
    EAGLE_LAUNCH_CHECK();
    return EAGLE_OK;
  }
  EAGLE_REQUIRE(workspace && ws_bytes >= need, EAGLE_EWORKSPACE);
  EAGLE_REQUIRE(((uintptr_t)workspace & 255) == 0, EAGLE_EINVAL);
  const int chunks = lp_chunks(V);
  int32_t* ctr = (int32_t*)workspace;
  selkey_t* cand = (selkey_t*)((char*)workspace + lp_ctr_bytes(T));
  const bool vec = (V & 3) == 0 && (((uintptr_t)logits | (uintptr_t)out) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(lp_chunk_kernel<true>, dim3(T, chunks), dim3(kLcThreads), 0, stream, logits,
                       V, k, inv_t, top_p, out, kept, cand, ctr);
  else
    hipLaunchKernelGGL(lp_chunk_kernel<false>, dim3(T, chunks), dim3(kLcThreads), 0, stream, logits,
                       V, k, inv_t, top_p, out, kept, cand, ctr);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
