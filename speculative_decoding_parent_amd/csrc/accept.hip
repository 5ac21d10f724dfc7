// Acceptance of the longest verified path through the draft tree.
//
// Sources: "EAGLE-2: Feature-Level Speculative Decoding Guide", Key
// Architectural Mechanics 3 - a greedy or sampling verifier walks the tree
// from the root and accepts matching tokens until the first discrepancy;
// The Problem 1 and "Support Eagle-3 Speculative Decoding in llama.cpp"
// (opening post) - speculative sampling's accept/reject rule.
//
// GREEDY: one thread per node walks to the root checking that every step holds
// the target's choice; the deepest fully matching node (lowest index on ties)
// ends the path.
//
// SAMPLE: the walk itself is sequential and touches at most depth+1 rows, but
// each row needs fp64 softmax mass over the whole vocabulary.  A grid kernel
// first reduces every row in 4096-token chunks (chunk max and fp64
// sum of exp((l - chunk max) / temperature)), so the single-workgroup walk
// only combines ~32 chunk sums per visited node (one wave, in parallel) and
// rescans one 4096-token chunk for the inverse-CDF draw.
#include <algorithm>

#include "common.h"

namespace eagle {

constexpr int kAcceptChunk = 4096;

// e^x in fp64 for x <= 0 (the exponents here are (l - max) / temperature).
// Cody-Waite reduction x = k ln2 + r with ln2 split into a head with
// trailing zero bits and a tail, so k ln2_hi is exact and |r| <= ln2 / 2;
// e^r by its Taylor series to degree 12 (remainder < 2e-16 on that range),
// then scaled by 2^k.  Within a few ulp of the correctly rounded value;
// 0 below -745.2 (and for -inf).
__device__ __forceinline__ double exp_nonpos(double x) {
  constexpr double kLn2Hi = 6.93147180369123816490e-01;
  constexpr double kLn2Lo = 1.90821492927058770002e-10;
  constexpr double kLog2e = 1.4426950408889634;
  if (!(x > -745.2)) return 0.0;
  const double k = rint(x * kLog2e);
  double r = fma(-k, kLn2Hi, x);
  r = fma(-k, kLn2Lo, r);
  double p = 2.08767569878681e-09;
  p = fma(p, r, 2.505210838544172e-08);
  p = fma(p, r, 2.755731922398589e-07);
  p = fma(p, r, 2.7557319223985893e-06);
  p = fma(p, r, 2.48015873015873e-05);
  p = fma(p, r, 0.0001984126984126984);
  p = fma(p, r, 0.001388888888888889);
  p = fma(p, r, 0.008333333333333333);
  p = fma(p, r, 0.041666666666666664);
  p = fma(p, r, 0.16666666666666666);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)k);
}

// ---------------------------------------------------------------- greedy

__global__ __launch_bounds__(256) void accept_greedy_kernel(
    int T, const int32_t* __restrict__ token, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ top1, int top1_stride, int max_path, int32_t* __restrict__ path,
    int32_t* __restrict__ n_acc, int32_t* __restrict__ bonus, int32_t* __restrict__ status) {
  __shared__ int32_t par[EAGLE_MAX_TREE];
  __shared__ int32_t tk[EAGLE_MAX_TREE];
  __shared__ int32_t t1[EAGLE_MAX_TREE];
  __shared__ int32_t key[EAGLE_MAX_TREE];
  const int tid = threadIdx.x;
  for (int i = tid; i < T; i += blockDim.x) {
    par[i] = parent[i];
    tk[i] = token[i];
    t1[i] = top1[(int64_t)i * top1_stride];
  }
  __syncthreads();
  for (int i = tid; i < T; i += blockDim.x) {
    // key = depth * 256 + (255 - i) for accepted nodes, -1 otherwise: the
    // largest key is the deepest accepted node with the lowest index.
    int ok = 1;
    int d = 0;
    int j = i;
    if (i == 0 && par[0] != -1) set_status(status, EAGLE_DEV_BAD_ROOT);
    while (j != 0) {
      const int p = par[j];
      if (p < 0 || p >= j) {
        set_status(status, p == -1 ? EAGLE_DEV_BAD_ROOT : EAGLE_DEV_BAD_PARENT);
        ok = 0;
        break;
      }
      if (tk[j] != t1[p]) ok = 0;
      ++d;
      j = p;
    }
    key[i] = ok ? d * 256 + (255 - i) : -1;
  }
  __syncthreads();
  if (tid < 64) {
    int best = -1;
    for (int i = tid; i < T; i += 64) best = max(best, key[i]);
    best = wave_max_i(best);
    if (tid == 0) {
      const int end = best < 0 ? 0 : 255 - (best & 255);
      const int depth = best < 0 ? 0 : (best >> 8);
      // path[0..depth] from the root; cut if it does not fit
      int u = end;
      for (int s = depth; s >= 0; --s) {
        if (s < max_path) path[s] = u;
        u = s > 0 ? par[u] : u;
      }
      for (int s = depth + 1; s < max_path; ++s) path[s] = -1;
      if (depth + 1 > max_path) set_status(status, EAGLE_DEV_PATH_TRUNC);
      *n_acc = min(depth, max_path - 1);
      *bonus = t1[end];
    }
  }
}

// ---------------------------------------------------------------- sampling

// Per (row, chunk): chunk max m_c (fp32, exact) and s_c = sum over the chunk of
// exp(((double)l - m_c) / temperature) in fp64 (the division taken as a
// product with the fp64 reciprocal: at most one ulp of the exponent, and
// exact for temperature 1).
// Rows [0, T0) of the grid read logits0 and write ws0, the rest logits1 and
// ws1 (one launch for the target's and the draft's rows).
__global__ __launch_bounds__(256) void accept_row_stats_kernel(
    const float* __restrict__ logits0, double* __restrict__ ws0, int T0,
    const float* __restrict__ logits1, double* __restrict__ ws1, int V, double itemp,
    int nchunk) {
  constexpr int PER = kAcceptChunk / 256;  // logits per thread, held in registers
  const int c = blockIdx.x;
  const bool second = (int)blockIdx.y >= T0;
  const int t = second ? (int)blockIdx.y - T0 : (int)blockIdx.y;
  const float* row = (second ? logits1 : logits0) + (size_t)t * V;
  double* ws = second ? ws1 : ws0;
  const int lo = c * kAcceptChunk;
  const int hi = min(V, lo + kAcceptChunk);
  __shared__ float smax[4];
  __shared__ double ssum[4];
  float x[PER];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int v = lo + (int)threadIdx.x + 256 * j;
    x[j] = v < hi ? row[v] : -INFINITY;
    m = fmaxf(m, x[j]);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) smax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(smax[0], smax[1]), fmaxf(smax[2], smax[3]));
  double s = 0.0;
  const double md = (double)m;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int v = lo + (int)threadIdx.x + 256 * j;
    if (v < hi) s += exp_nonpos(((double)x[j] - md) * itemp);
  }
  s = wave_sum_d(s);
  if ((threadIdx.x & 63) == 0) ssum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double* o = ws + ((size_t)t * nchunk + c) * 2;
    o[0] = md;
    o[1] = ((ssum[0] + ssum[1]) + ssum[2]) + ssum[3];
  }
}

// Block-wide reduction; `red` holds one slot per wave.  The leading barrier
// lets the same `red` be reused by back-to-back calls.
template <typename V, typename Op>
__device__ __forceinline__ V block_reduce(V v, V* red, Op op) {
  v = wave_reduce(v, op);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  V r = red[0];
  const int nw = blockDim.x >> 6;
  for (int i = 1; i < nw; ++i) r = op(r, red[i]);
  return r;
}

__global__ __launch_bounds__(1024) void accept_sample_kernel(
    int T, const int32_t* __restrict__ token, const int32_t* __restrict__ parent,
    const float* __restrict__ logits, int V, double itemp, const float* __restrict__ U,
    int nchunk, const double* __restrict__ ws, int max_path, int32_t* __restrict__ path,
    int32_t* __restrict__ n_acc, int32_t* __restrict__ bonus, int32_t* __restrict__ status) {
  __shared__ int32_t par[EAGLE_MAX_TREE];
  __shared__ int32_t tk[EAGLE_MAX_TREE];
  __shared__ int32_t rej[EAGLE_MAX_TREE];
  __shared__ double pxs[EAGLE_MAX_TREE];
  __shared__ double dred[16];
  __shared__ int ired[16];
  __shared__ double sh_m, sh_target, sh_run;
  __shared__ int sh_u, sh_nrej, sh_moved, sh_chunk;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  for (int i = tid; i < T; i += blockDim.x) {
    int p = parent[i];
    const int x = token[i];
    if (i == 0 ? p != -1 : (p < 0 || p >= i)) {
      set_status(status, (i == 0 || p == -1) ? EAGLE_DEV_BAD_ROOT : EAGLE_DEV_BAD_PARENT);
      p = i == 0 ? -1 : 0;
    }
    if (x < 0 || x >= V) set_status(status, EAGLE_DEV_BAD_TOKEN);
    par[i] = p;
    tk[i] = min(max(x, 0), V - 1);
  }
  if (tid == 0) sh_u = 0;
  __syncthreads();

  // ---- the walk: one accept/reject pass over the children of each node.
  // Wave 0 combines the node's chunk statistics and weighs every child in
  // parallel; lane 0 then takes the decisions in child order.
  int depth = 0;
  for (;;) {
    if (tid < 64) {
      const int u = sh_u;
      const float* row = logits + (size_t)u * V;
      const double* st = ws + (size_t)u * nchunk * 2;
      double m = -INFINITY;
      for (int c = lane; c < nchunk; c += 64) m = fmax(m, st[2 * c]);
      m = wave_max_d(m);
      double z = 0.0;
      for (int c = lane; c < nchunk; c += 64) z += st[2 * c + 1] * exp_nonpos((st[2 * c] - m) * itemp);
      z = wave_sum_d(z);
      uint64_t kids[EAGLE_MAX_TREE / 64];
#pragma unroll
      for (int q = 0; q < EAGLE_MAX_TREE / 64; ++q) {
        const int c = 64 * q + lane;
        const bool is = c > u && c < T && par[c] == u;
        if (is) pxs[c] = exp_nonpos(((double)row[tk[c]] - m) * itemp);
        kids[q] = __builtin_amdgcn_ballot_w64(is);
      }
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) {
        double zres = z;
        int nrej = 0;
        int moved = 0;
        for (int q = 0; q < EAGLE_MAX_TREE / 64 && !moved; ++q) {
          uint64_t b = kids[q];
          while (b && !moved) {
            const int c = 64 * q + __builtin_ctzll(b);
            b &= b - 1;
            const int x = tk[c];
            bool seen = false;
            for (int r = 0; r < nrej; ++r) seen |= rej[r] == x;
            if (seen) continue;
            const double px = pxs[c];
            if ((double)U[c] * zres < px) {
              moved = 1;
              sh_u = c;
            } else {
              rej[nrej++] = x;
              zres = zres - px;
            }
          }
        }
        sh_m = m;
        sh_nrej = nrej;
        sh_moved = moved;
        sh_target = (double)U[T + u] * zres;
      }
      __builtin_amdgcn_wave_barrier();
      if (!sh_moved) {
        // the residual draw starts in the first chunk whose running
        // non-rejected mass passes the target
        const int nrej = sh_nrej;
        const double target = sh_target;
        double run = 0.0;
        int chunk = nchunk - 1;
        double before = run;
        for (int c0 = 0; c0 < nchunk; c0 += 64) {
          const int c = c0 + lane;
          double mass = 0.0;
          if (c < nchunk) {
            mass = st[2 * c + 1] * exp_nonpos((st[2 * c] - m) * itemp);
            for (int r = 0; r < nrej; ++r)
              if (rej[r] / kAcceptChunk == c) mass -= exp_nonpos(((double)row[rej[r]] - m) * itemp);
          }
          double incl = mass;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
          }
          // (if no chunk passes, the draw starts in the last one)
          const int lastw = nchunk - 1 - c0;
          if (lastw < 64) before = run + __shfl(incl - mass, lastw);
          const uint64_t pass = __builtin_amdgcn_ballot_w64(c < nchunk && run + incl > target);
          if (pass) {
            const int w = __builtin_ctzll(pass);
            chunk = c0 + w;
            before = run + __shfl(incl - mass, w);
            break;
          }
          run += __shfl(incl, 63);
        }
        if (lane == 0) {
          sh_chunk = chunk;
          sh_run = before;
        }
      }
    }
    __syncthreads();
    if (!sh_moved) break;
    ++depth;
    if (tid == 0 && depth < max_path) path[depth] = sh_u;
    __syncthreads();
  }

  // ---- residual draw at the last node: inverse CDF in token order
  const int u = sh_u;
  const float* row = logits + (size_t)u * V;
  const double m = sh_m;
  const double target = sh_target;
  const int nrej = sh_nrej;
  double run = sh_run;
  int found = INT_MAX;
  int lastpos = -1;
  for (int c = sh_chunk; c < nchunk; ++c) {
    const int lo = c * kAcceptChunk;
    const int hi = min(V, lo + kAcceptChunk);
    const int v0 = lo + tid * 4;          // 1024 threads x 4 tokens = one chunk
    double q[4];
    double mine = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v0 + e;
      double pv = 0.0;
      if (v < hi) {
        bool r = false;
        for (int j = 0; j < nrej; ++j) r |= rej[j] == v;
        pv = r ? 0.0 : exp_nonpos(((double)row[v] - m) * itemp);
      }
      q[e] = pv;
      mine += pv;
    }
    double incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == 63) dred[tid >> 6] = incl;
    __syncthreads();
    double off = run;
    for (int w = 0; w < (tid >> 6); ++w) off += dred[w];
    double total = 0.0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) total += dred[w];
    double cum = off + (incl - mine);
    int hit = INT_MAX;
    int last = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (q[e] > 0.0) {
        last = v0 + e;
        cum += q[e];
        if (hit == INT_MAX && cum > target) hit = v0 + e;
      }
    }
    hit = block_reduce(hit, ired, [](int a, int b) { return min(a, b); });
    last = block_reduce(last, ired, [](int a, int b) { return max(a, b); });
    lastpos = max(lastpos, last);
    if (hit != INT_MAX) {
      found = hit;
      break;
    }
    run = run + total;
  }
  if (tid == 0) {
    const int b = found != INT_MAX ? found : max(lastpos, 0);
    for (int s = depth + 1; s < max_path; ++s) path[s] = -1;
    path[0] = 0;
    if (depth + 1 > max_path) set_status(status, EAGLE_DEV_PATH_TRUNC);
    *n_acc = min(depth, max_path - 1);
    *bonus = b;
  }
}

// ---------------------------------------------------------------- draft q

// Speculative sampling with the draft's distribution (recursive rejection
// sampling over the children of each node, drawn from q without
// replacement), spread over the whole GPU.  G workgroups (one per CU, all
// resident at once) each own a contiguous chunk of the vocabulary and walk
// the tree together: every workgroup takes every decision itself from the
// same data in the same order, so they agree without exchanging decisions,
// and they meet at a grid barrier only where a decision needs a sum over the
// vocabulary.  At a visited node u:
//   * one barrier combines the chunks' (max, sum e^((l - max) / t)) of the
//     target and draft rows into Zp, Zq; each thread then holds
//     p1(y) = e^((l_y - M) / t) / Zp and q1(y) for its tokens in fp64;
//   * child i (ascending index) with token x, not rejected before, is
//     accepted iff U[c] q_i(x) < p_i(x).  Every workgroup evaluates p_i(x) and
//     q_i(x) at x alone: p1(x), q1(x) from the logits, then the node's
//     earlier rejections replayed (p <- max(p - q, 0) / Z, q_i = q1 / D_i with
//     D_i = 1 - the rejected draft mass);
//   * a rejection makes every thread form max(p_i(y) - q_i(y), 0) for its
//     tokens; one barrier gives their sum Z_(i+1); x's draft mass leaves D;
//   * with no child accepted, the bonus is the smallest token whose running
//     sum of p exceeds U[T + u] sum(p): one barrier for the chunk sums (each
//     workgroup then scans its own chunk in token order), one for the
//     crossing (the lowest token found, or the last token with mass when
//     rounding leaves none).
// The workgroups meet at a barrier with a coordinator: each publishes a
// record (device-coherent stores) and then its arrival flag; workgroup 0
// waits for every flag, combines the records in a fixed order, publishes the
// result and a release flag, which the others wait for.  No atomics, so the
// cost of a barrier does not grow with G.  Flags carry a generation number
// that workgroup 0 advances at the end of every call (so stale flags never
// match: flags are compared for equality, and a workgroup cannot publish
// barrier e + 1's flag before barrier e is released) and the barrier's index
// within the call.  Every wait is bounded
// (kQSpinLimit polls): a barrier that never fills sets EAGLE_DEV_TIMEOUT and
// the walk stops instead of hanging.
constexpr int kQG = 256;           // workgroups (at most; one per CU)
constexpr int kQT = 256;           // threads per workgroup
constexpr int kQE = 8;             // vocabulary entries per thread, at most
constexpr int kQWv = kQT / 64;
constexpr uint32_t kQSpinLimit = 1u << 20;   // polls per barrier (about a second)

struct QGridParams {
  int T, V, G, C, E;               // C: chunk per workgroup, E: entries per thread
  const int32_t* token;
  const int32_t* parent;
  const float* tl;
  const float* dl;
  double itemp;
  const float* U;
  int max_path;
  int32_t* path;
  int32_t* n_acc;
  int32_t* bonus;
  int32_t* status;
  int32_t* sync;                   // [0] generation, [32] release flag, [64 + w] arrival flags
  double* rec;                     // [2][G][4] published records, alternating per barrier
  double* res;                     // [2][8 + G] combined results (+ per-chunk prefix sums)
};

enum { kQStats = 0, kQSum = 1, kQScan = 2 };

// Sum (or max) over the workgroup in a fixed order; every thread gets it.
__device__ __forceinline__ double q_wg_sum(double v, double* red) {
  v = wave_sum_d(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kQWv; ++w) s += red[w];
  return s;
}
__device__ __forceinline__ double q_wg_max(double v, double* red) {
  v = wave_max_d(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double m = -INFINITY;
#pragma unroll
  for (int w = 0; w < kQWv; ++w) m = fmax(m, red[w]);
  return m;
}

__global__ __launch_bounds__(kQT) void accept_q_grid_kernel(QGridParams p) {
  __shared__ int32_t par[EAGLE_MAX_TREE];
  __shared__ int32_t tk[EAGLE_MAX_TREE];
  __shared__ int32_t kid[EAGLE_MAX_TREE];
  __shared__ int32_t rej[EAGLE_MAX_TREE];
  __shared__ double hz[EAGLE_MAX_TREE];   // 1 / Z after each rejection at this node
  __shared__ double hd[EAGLE_MAX_TREE];   // 1 / D before each rejection (0: no draft mass)
  __shared__ double red[kQWv];
  __shared__ double xch[kQG][4];          // workgroup 0: the G records
  __shared__ double res[4];               // a barrier's combined result
  __shared__ double sh_before;
  __shared__ int sh_ok, sh_nk;
  const int tid = threadIdx.x;
  const int w = blockIdx.x;
  const int G = p.G, V = p.V, T = p.T, E = p.E;
  const int c0 = w * p.C;
  const int c1 = min(c0 + p.C, V);
  const int e0 = c0 + tid * E;            // this thread's tokens [e0, e0 + E) within [c0, c1)
  const bool lead = w == 0;
  int epoch = 0;
  bool alive = true;

  for (int i = tid; i < T; i += kQT) {
    int pp = p.parent[i];
    const int x = p.token[i];
    if (i == 0 ? pp != -1 : (pp < 0 || pp >= i)) {
      if (lead) set_status(p.status, (i == 0 || pp == -1) ? EAGLE_DEV_BAD_ROOT : EAGLE_DEV_BAD_PARENT);
      pp = i == 0 ? -1 : 0;
    }
    if (x < 0 || x >= V) {
      if (lead) set_status(p.status, EAGLE_DEV_BAD_TOKEN);
    }
    par[i] = pp;
    tk[i] = min(max(x, 0), V - 1);
  }
  __syncthreads();

  // Barrier: publish this workgroup's record (a, b, c, d), meet the others,
  // and receive the combination of all G records in res[]: kQStats -> (M, Zp,
  // Md, Zq) from chunk (max, sum) pairs; kQSum -> the sum of the a's; kQScan
  // -> (the sum of the a's, the largest b) and, in sh_before, the sum of the
  // a's of the chunks before this one.  false: a wait expired.
  const int gen = __hip_atomic_load(p.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto exchange = [&](int kind, double a, double b, double c, double d) -> bool {
    const int slot = epoch & 1;
    const int want = (gen << 10) | (epoch + 1);
    const __amdgpu_buffer_rsrc_t rrs = dev_rsrc(p.rec + (size_t)slot * G * 4, (size_t)G * 32);
    const __amdgpu_buffer_rsrc_t ors = dev_rsrc(p.res + (size_t)slot * (8 + G), (size_t)(8 + G) * 8);
    ++epoch;
    if (tid == 0) {
      st_dev4(rrs, (uint32_t)(w * 32), __builtin_bit_cast(f32x4, make_double2(a, b)));
      st_dev4(rrs, (uint32_t)(w * 32 + 16), __builtin_bit_cast(f32x4, make_double2(c, d)));
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));   // the record lands before the flag
      __hip_atomic_store(p.sync + 64 + w, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int ok = 1;
    if (lead) {
      // workgroup 0: every arrival, then every record, combined in order
      if (tid < G) {
        uint32_t spins = 0;
        while (__hip_atomic_load(p.sync + 64 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
               want) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins >= kQSpinLimit) {
            ok = 0;
            break;
          }
        }
      }
      if (!ok) set_status(p.status, EAGLE_DEV_TIMEOUT);
      if (tid == 0) sh_ok = 1;
      __syncthreads();
      if (!ok) sh_ok = 0;
      __syncthreads();
      if (!sh_ok) return false;
      double ra = 0.0, rb = 0.0, rc = 0.0, rd = 0.0;
      if (tid < G) {
        const double2 x = __builtin_bit_cast(double2, ld_dev4(rrs, (uint32_t)(tid * 32)));
        const double2 y = __builtin_bit_cast(double2, ld_dev4(rrs, (uint32_t)(tid * 32 + 16)));
        ra = x.x; rb = x.y; rc = y.x; rd = y.y;
        xch[tid][0] = ra; xch[tid][1] = rb; xch[tid][2] = rc; xch[tid][3] = rd;
      }
      double o0 = 0.0, o1 = 0.0, o2 = 0.0, o3 = 0.0;
      if (kind == kQStats) {
        o0 = q_wg_max(tid < G ? ra : -INFINITY, red);
        o2 = q_wg_max(tid < G ? rc : -INFINITY, red);
        o1 = q_wg_sum(tid < G && rb > 0.0 ? rb * exp_nonpos((ra - o0) * p.itemp) : 0.0, red);
        o3 = q_wg_sum(tid < G && rd > 0.0 ? rd * exp_nonpos((rc - o2) * p.itemp) : 0.0, red);
      } else if (kind == kQSum) {
        o0 = q_wg_sum(tid < G ? ra : 0.0, red);
      } else {
        o1 = q_wg_max(tid < G ? rb : -1.0, red);
        __syncthreads();                          // xch is complete
        if (tid == 0) {                           // prefix in chunk order
          double run = 0.0;
          for (int v = 0; v < G; ++v) {
            const double nx = run + xch[v][0];
            xch[v][1] = run;
            run = nx;
          }
          red[0] = run;
        }
        __syncthreads();
        o0 = red[0];
        if (tid < G) st_dev2(ors, (uint32_t)((8 + tid) * 8),
                             __builtin_bit_cast(u32x2, xch[tid][1]));
        if (tid == 0) sh_before = xch[0][1];
      }
      if (tid == 0) {
        st_dev4(ors, 0, __builtin_bit_cast(f32x4, make_double2(o0, o1)));
        st_dev4(ors, 16, __builtin_bit_cast(f32x4, make_double2(o2, o3)));
        res[0] = o0; res[1] = o1; res[2] = o2; res[3] = o3;
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));   // results land before the release
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(p.sync + 32, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      return true;
    }
    if (tid == 0) {
      uint32_t spins = 0;
      while (__hip_atomic_load(p.sync + 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins >= kQSpinLimit) {
          ok = 0;
          break;
        }
      }
      if (!ok) set_status(p.status, EAGLE_DEV_TIMEOUT);
      if (ok) {
        const double2 x = __builtin_bit_cast(double2, ld_dev4(ors, 0));
        const double2 y = __builtin_bit_cast(double2, ld_dev4(ors, 16));
        res[0] = x.x; res[1] = x.y; res[2] = y.x; res[3] = y.y;
        if (kind == kQScan)
          sh_before = __builtin_bit_cast(double, ld_dev2(ors, (uint32_t)((8 + w) * 8)));
      }
      sh_ok = ok;
    }
    __syncthreads();
    return sh_ok != 0;
  };

  double pv[kQE], qv[kQE];
  int u = 0, depth = 0;
  if (lead && tid == 0) p.path[0] = 0;
  for (;;) {
    const float* lrow = p.tl + (size_t)u * V;
    const float* drow = p.dl + (size_t)u * V;
    // this chunk's row statistics
    float lf[kQE], df[kQE];
    float ml = -INFINITY, md = -INFINITY;
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      const int y = e0 + e;
      const bool in = e < E && y < c1;
      lf[e] = in ? lrow[y] : -INFINITY;
      df[e] = in ? drow[y] : -INFINITY;
      ml = fmaxf(ml, lf[e]);
      md = fmaxf(md, df[e]);
    }
    const double wml = q_wg_max((double)ml, red);
    const double wmd = q_wg_max((double)md, red);
    double sp = 0.0, sq = 0.0;
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      if (e < E && e0 + e < c1) {
        sp += exp_nonpos(((double)lf[e] - wml) * p.itemp);
        sq += exp_nonpos(((double)df[e] - wmd) * p.itemp);
      }
    }
    const double wsp = q_wg_sum(sp, red);
    const double wsq = q_wg_sum(sq, red);
    if (!exchange(kQStats, wml, wsp, wmd, wsq)) {
      alive = false;
      break;
    }
    const double M = res[0], zp = res[1], Md = res[2], zq = res[3];
    const double izp = 1.0 / zp;
    const double izq = 1.0 / zq;
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      const bool in = e < E && e0 + e < c1;
      pv[e] = in ? exp_nonpos(((double)lf[e] - M) * p.itemp) * izp : 0.0;
      qv[e] = in ? exp_nonpos(((double)df[e] - Md) * p.itemp) * izq : 0.0;
    }
    if (tid == 0) {
      int n = 0;
      for (int c = u + 1; c < T; ++c)
        if (par[c] == u) kid[n++] = c;
      sh_nk = n;
    }
    __syncthreads();
    const int nk = sh_nk;
    int nrej = 0;
    double D = 1.0;                          // draft mass not yet rejected at u
    int next = -1;
    for (int i = 0; i < nk; ++i) {
      const int c = kid[i];
      const int x = tk[c];
      bool seen = false;
      for (int r = 0; r < nrej; ++r) seen |= rej[r] == x;
      if (seen) continue;                    // a draw never repeats a token
      // p_i(x), q_i(x) at x alone, replaying this node's rejections
      const double q1x = exp_nonpos(((double)drow[x] - Md) * p.itemp) * izq;
      double px = exp_nonpos(((double)lrow[x] - M) * p.itemp) * izp;
      for (int r = 0; r < nrej; ++r) px = fmax(px - q1x * hd[r], 0.0) * hz[r];
      const double iD = D > 0.0 ? 1.0 / D : 0.0;
      const double qx = q1x * iD;
      if ((double)p.U[c] * qx < px) {
        next = c;
        break;
      }
      // rejected: p <- max(p - q, 0) / Z, over the vocabulary (the same
      // operations as the replay above)
      double s = 0.0;
#pragma unroll
      for (int e = 0; e < kQE; ++e) {
        const double t = fmax(pv[e] - qv[e] * iD, 0.0);
        pv[e] = t;
        s += t;
      }
#pragma unroll
      for (int e = 0; e < kQE; ++e)
        if (e0 + e == x) qv[e] = 0.0;        // x leaves q after this step's update
      const double ws = q_wg_sum(s, red);
      if (!exchange(kQSum, ws, 0.0, 0.0, 0.0)) {
        alive = false;
        break;
      }
      const double iz = 1.0 / res[0];
      if (tid == 0) {
        hd[nrej] = iD;
        hz[nrej] = iz;
        rej[nrej] = x;
      }
#pragma unroll
      for (int e = 0; e < kQE; ++e) pv[e] *= iz;
      D -= q1x;
      ++nrej;
      __syncthreads();
    }
    if (!alive) break;
    if (next >= 0) {
      ++depth;
      if (lead && tid == 0) {
        if (depth < p.max_path) p.path[depth] = next;
        else set_status(p.status, EAGLE_DEV_PATH_TRUNC);
      }
      u = next;
      continue;
    }
    // bonus: the smallest token whose running sum of p exceeds U[T + u] sum(p)
    double own = 0.0;
#pragma unroll
    for (int e = 0; e < kQE; ++e) own += pv[e];
    // exclusive prefix of the threads' sums, in thread order
    __shared__ double tsum[kQT];
    tsum[tid] = own;
    __syncthreads();
    if (tid == 0) {
      double run = 0.0;
      for (int t = 0; t < kQT; ++t) {
        const double nx = run + tsum[t];
        tsum[t] = run;
        run = nx;
      }
      red[0] = run;
    }
    __syncthreads();
    const double wtot = red[0];
    const double tpre = tsum[tid];
    int last = -1;
#pragma unroll
    for (int e = 0; e < kQE; ++e)
      if (pv[e] > 0.0) last = e0 + e;
    last = (int)q_wg_max((double)last, red);
    if (!exchange(kQScan, wtot, (double)last, 0.0, 0.0)) {
      alive = false;
      break;
    }
    const double total = res[0];
    const int lastall = (int)res[1];
    const double before = sh_before;
    const double target = (double)p.U[T + u] * total;
    // Chunk boundaries are consistent (each chunk starts where the previous
    // one's prefix ends), so exactly one chunk holds the crossing when
    // target < total; it reports the first of its tokens whose running sum
    // exceeds target (the last token of the chunk with mass if rounding
    // inside the chunk leaves none).  Otherwise rounding left no crossing at
    // all: the last token with mass.
    if (target < total && before <= target && target < before + wtot) {
      int hit = 0x7fffffff;
      double run = before + tpre;
#pragma unroll
      for (int e = 0; e < kQE; ++e) {
        const double nx = run + pv[e];
        if (hit == 0x7fffffff && e < E && e0 + e < c1 && nx > target) hit = e0 + e;
        run = nx;
      }
      hit = -(int)q_wg_max(-(double)hit, red);    // lowest in the workgroup
      if (hit == 0x7fffffff) hit = max(last, 0);
      if (tid == 0) p.bonus[0] = hit;
    } else if (!(target < total) && lead && tid == 0) {
      p.bonus[0] = max(lastall, 0);
    }
    if (lead && tid == 0) {
      p.n_acc[0] = min(depth, p.max_path - 1);
      for (int d = depth + 1; d < p.max_path; ++d) p.path[d] = -1;
    }
    break;
  }
  // a new generation for the next call: its flags never match this call's
  if (lead && tid == 0)
    __hip_atomic_store(p.sync, (gen + 1) & 0x1fffff, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  (void)alive;
}

}  // namespace eagle

extern "C" size_t eagle_accept_workspace(int32_t T, int32_t V) {
  if (T < 1 || V < 1) return 0;
  const size_t nchunk = ((size_t)V + eagle::kAcceptChunk - 1) / eagle::kAcceptChunk;
  return (size_t)T * nchunk * 2 * sizeof(double);
}

extern "C" int eagle_accept(int32_t mode, int32_t T, const int32_t* node_token,
                            const int32_t* node_parent, const int32_t* target_top1,
                            int32_t top1_stride, const float* target_logits, int32_t V,
                            float temperature,
                            const float* uniforms, int32_t max_path, int32_t* path,
                            int32_t* n_accepted, int32_t* bonus_token, void* workspace,
                            size_t ws_bytes, int32_t* dev_status, hipStream_t stream) {
  EAGLE_REQUIRE(node_token && node_parent && path && n_accepted && bonus_token, EAGLE_EINVAL);
  EAGLE_REQUIRE(T >= 1 && T <= EAGLE_MAX_TREE && max_path >= 1, EAGLE_EINVAL);
  if (mode == EAGLE_GREEDY) {
    EAGLE_REQUIRE(target_top1 && top1_stride >= 1, EAGLE_EINVAL);
    hipLaunchKernelGGL(eagle::accept_greedy_kernel, dim3(1), dim3(256), 0, stream, T, node_token,
                       node_parent, target_top1, top1_stride, max_path, path, n_accepted,
                       bonus_token, dev_status);
  } else if (mode == EAGLE_SAMPLE) {
    EAGLE_REQUIRE(target_logits && uniforms && V >= 1, EAGLE_EINVAL);
    EAGLE_REQUIRE(temperature > 0.0f && temperature <= 3.0e38f, EAGLE_EINVAL);
    EAGLE_REQUIRE(workspace && ((uintptr_t)workspace & 7) == 0, EAGLE_EINVAL);
    EAGLE_REQUIRE(ws_bytes >= eagle_accept_workspace(T, V), EAGLE_EWORKSPACE);
    const int nchunk = (V + eagle::kAcceptChunk - 1) / eagle::kAcceptChunk;
    const double itemp = 1.0 / (double)temperature;
    hipLaunchKernelGGL(eagle::accept_row_stats_kernel, dim3(nchunk, T), dim3(256), 0, stream,
                       target_logits, (double*)workspace, T, target_logits, (double*)workspace, V,
                       itemp, nchunk);
    EAGLE_LAUNCH_CHECK();
    hipLaunchKernelGGL(eagle::accept_sample_kernel, dim3(1), dim3(1024), 0, stream, T,
                       node_token, node_parent, target_logits, V, itemp, uniforms, nchunk,
                       (const double*)workspace, max_path, path, n_accepted, bonus_token,
                       dev_status);
  } else {
    return EAGLE_EINVAL;
  }
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

// Compute units of the current device: the general-q walk needs its whole
// grid resident at once, one workgroup per CU.
static int q_device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return eagle::kQG;
  if (!cached[dev]) {
    int n = 0;
    cached[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                          hipSuccess && n > 0 ? n : eagle::kQG;
  }
  return cached[dev];
}

extern "C" size_t eagle_accept_q_workspace(int32_t T, int32_t V) {
  if (T < 1 || V < 1) return 0;
  return 2048 + (size_t)2 * eagle::kQG * 4 * sizeof(double) +
         (size_t)2 * (8 + eagle::kQG) * sizeof(double);
}

extern "C" int eagle_accept_q(int32_t T, const int32_t* node_token, const int32_t* node_parent,
                              const float* target_logits, const float* draft_logits, int32_t V,
                              float temperature, const float* uniforms, int32_t max_path,
                              int32_t* path, int32_t* n_accepted, int32_t* bonus_token,
                              void* workspace, size_t ws_bytes, int32_t* dev_status,
                              hipStream_t stream) {
  EAGLE_REQUIRE(node_token && node_parent && target_logits && draft_logits && uniforms, EAGLE_EINVAL);
  EAGLE_REQUIRE(path && n_accepted && bonus_token, EAGLE_EINVAL);
  EAGLE_REQUIRE(T >= 1 && T <= EAGLE_MAX_TREE && max_path >= 1 && V >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(temperature > 0.0f && temperature <= 3.0e38f, EAGLE_EINVAL);
  EAGLE_REQUIRE(workspace && ((uintptr_t)workspace & 255) == 0, EAGLE_EINVAL);
  EAGLE_REQUIRE(ws_bytes >= eagle_accept_q_workspace(T, V), EAGLE_EWORKSPACE);
  const int G = std::min(eagle::kQG, q_device_cus());
  const int C = (V + G - 1) / G;
  const int E = (C + eagle::kQT - 1) / eagle::kQT;
  EAGLE_REQUIRE(E <= eagle::kQE, EAGLE_EUNSUPPORTED);
  eagle::QGridParams p{};
  p.T = T; p.V = V; p.G = G; p.C = C; p.E = E;
  p.token = node_token; p.parent = node_parent; p.tl = target_logits; p.dl = draft_logits;
  p.itemp = 1.0 / (double)temperature;
  p.U = uniforms; p.max_path = max_path; p.path = path; p.n_acc = n_accepted;
  p.bonus = bonus_token; p.status = dev_status;
  p.sync = (int32_t*)workspace;                                  // 64 + kQG ints
  p.rec = (double*)((char*)workspace + 2048);                    // [2][G][4]
  p.res = p.rec + 2 * eagle::kQG * 4;                            // [2][8 + G]
  hipLaunchKernelGGL(eagle::accept_q_grid_kernel, dim3(G), dim3(eagle::kQT), 0, stream, p);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
