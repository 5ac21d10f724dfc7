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
  const bool under = !(x > -745.2);     // (no branch: callers evaluate many at once)
  x = under ? 0.0 : x;
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
  const double v = ldexp(p, (int)k);
  return under ? 0.0 : v;
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
// A barrier is an all-gather of tagged records: each workgroup stores its
// record (four doubles) as eight 64-bit words with device-coherent stores,
// the low half of each word carrying half of a value and the high half the
// barrier's tag; thread v of every workgroup polls record v until all eight
// of its tags match, and every workgroup then combines the G records itself
// in the same fixed order.  Aligned 64-bit accesses are single-copy atomic,
// so a word whose tag matches carries this barrier's value; one memory round
// trip after the last record lands, every workgroup has them all.  Records
// alternate between two slots (a workgroup writes barrier e + 2's record only
// after everyone has written barrier e + 1's, that is, after everyone has read
// barrier e's).  Tags hold a generation number that workgroup 0 advances at
// the end of every call (so records of earlier calls never match) and the
// barrier's index within the call.  Every wait is bounded
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
  int32_t* sync;                   // [0] generation
  uint64_t* rec;                   // [2][G][8] tagged records, alternating per barrier
};

enum { kQStats = 0, kQSum = 1, kQScan = 2 };

// Sums and maxima over the workgroup in a fixed order (every thread gets
// them); two values share one pair of barriers.
__device__ __forceinline__ double2 q_wg_sum2(double a, double b, double2* red) {
  a = wave_sum_d(a);
  b = wave_sum_d(b);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_double2(a, b);
  __syncthreads();
  double2 s = make_double2(0.0, 0.0);
#pragma unroll
  for (int w = 0; w < kQWv; ++w) {
    s.x += red[w].x;
    s.y += red[w].y;
  }
  return s;
}
__device__ __forceinline__ double2 q_wg_max2(double a, double b, double2* red) {
  a = wave_max_d(a);
  b = wave_max_d(b);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_double2(a, b);
  __syncthreads();
  double2 m = make_double2(-INFINITY, -INFINITY);
#pragma unroll
  for (int w = 0; w < kQWv; ++w) {
    m.x = fmax(m.x, red[w].x);
    m.y = fmax(m.y, red[w].y);
  }
  return m;
}
// Exclusive prefix sums of v in thread order, and in *total the sum of all.
// The additions follow a fixed pattern, so equal inputs give equal results
// in every workgroup.
__device__ __forceinline__ double q_wg_excl_scan(double v, double2* red, double* total) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  double x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  double ex = __shfl_up(x, 1, 64);
  if (lane == 0) ex = 0.0;
  __syncthreads();
  if (lane == 63) red[wv] = make_double2(x, 0.0);
  __syncthreads();
  double off = 0.0, tot = 0.0;
#pragma unroll
  for (int w = 0; w < kQWv; ++w) {
    if (w < wv) off += red[w].x;
    tot += red[w].x;
  }
  *total = tot;
  return off + ex;
}

__global__ __launch_bounds__(kQT) void accept_q_grid_kernel(QGridParams p) {
  constexpr int kWords = EAGLE_MAX_TREE / 64;
  __shared__ int32_t par[EAGLE_MAX_TREE];
  __shared__ int32_t tk[EAGLE_MAX_TREE];
  __shared__ uint64_t cmask[EAGLE_MAX_TREE][kWords];   // the children of each node, as bits
  __shared__ int32_t fc[EAGLE_MAX_TREE];  // the first child of each node (T: none)
  __shared__ double cp1[EAGLE_MAX_TREE];  // a child's p1 and q1 at its token (row of its
  __shared__ double cq1[EAGLE_MAX_TREE];  //   parent), and its uniform
  __shared__ float chu[EAGLE_MAX_TREE];
  __shared__ int32_t rej[EAGLE_MAX_TREE];
  __shared__ double hz[EAGLE_MAX_TREE];   // 1 / Z after each rejection at this node
  __shared__ double hd[EAGLE_MAX_TREE];   // 1 / D before each rejection (0: no draft mass)
  __shared__ double2 red[kQWv];
  __shared__ double xb[kQG + 1];          // chunk boundaries of the bonus draw
  __shared__ double xw[kQG];              // and the chunks' masses
  __shared__ double tb[kQT + 1];          // thread boundaries within this chunk
  __shared__ float sh_ub;
  __shared__ int sh_fail;
  const int tid = threadIdx.x;
  const int w = blockIdx.x;
  const int G = p.G, V = p.V, T = p.T, E = p.E;
  const int c0 = w * p.C;
  const int c1 = min(c0 + p.C, V);
  const int e0 = c0 + tid * E;            // this thread's tokens [e0, e0 + E) within [c0, c1)
  const bool lead = w == 0;               // writes the outputs
  int epoch = 0;

  if (tid == 0) sh_fail = 0;
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
  for (int i = tid; i < EAGLE_MAX_TREE * kWords; i += kQT) (&cmask[0][0])[i] = 0ull;
  for (int i = tid; i < EAGLE_MAX_TREE; i += kQT) fc[i] = T;
  __syncthreads();
  for (int c = 1 + tid; c < T; c += kQT) {
    atomicOr((unsigned long long*)&cmask[par[c]][c >> 6], 1ull << (c & 63));
    atomicMin(&fc[par[c]], c);
  }
  __syncthreads();

  // Barrier: publish this workgroup's record (a, b, c, d), wait for every
  // workgroup's record of the same barrier, and combine all G of them in a
  // fixed order (every workgroup computes the same result) into r:
  // kQStats -> (M, Zp, Md, Zq) from chunk (max, sum) pairs; kQSum -> the sum
  // of the a's; kQScan -> (the sum of the a's, the largest b), with the
  // chunk boundaries (running sums of the a's in chunk order) in xb[0..G]
  // and the a's in xw.
  // false: a wait expired.
  const int gen = __hip_atomic_load(p.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto exchange = [&](int kind, double a, double b, double c, double d, double (&r)[4]) -> bool {
    const int slot = epoch & 1;
    const uint32_t want = (uint32_t)((gen << 10) | (epoch + 1));
    const __amdgpu_buffer_rsrc_t rrs = dev_rsrc(p.rec + (size_t)slot * G * 8, (size_t)G * 64);
    ++epoch;
    if (tid < 4) {
      // word 2 k + h of the record: half h of value k below, the tag above
      const double v = tid == 0 ? a : tid == 1 ? b : tid == 2 ? c : d;
      const uint64_t bits = __builtin_bit_cast(uint64_t, v);
      st_dev4(rrs, (uint32_t)(w * 64 + tid * 16),
              __builtin_bit_cast(f32x4, u32x4{(uint32_t)bits, want, (uint32_t)(bits >> 32), want}));
    }
    // thread v polls record v until all eight of its tags are this barrier's
    double rv[4] = {0.0, 0.0, 0.0, 0.0};
    if (tid < G) {
      uint32_t spins = 0;
      for (;;) {
        u32x4 x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          x[k] = __builtin_bit_cast(u32x4, ld_dev4(rrs, (uint32_t)(tid * 64 + k * 16)));
        bool all = true;
#pragma unroll
        for (int k = 0; k < 4; ++k) all = all && x[k][1] == want && x[k][3] == want;
        if (all) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            rv[k] = __builtin_bit_cast(double, ((uint64_t)x[k][2] << 32) | x[k][0]);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");   // the next poll reloads the record
        if (++spins >= kQSpinLimit) {
          set_status(p.status, EAGLE_DEV_TIMEOUT);
          sh_fail = 1;
          break;
        }
      }
    }
    __syncthreads();
    if (sh_fail) return false;
    const bool in = tid < G;
    if (kind == kQStats) {
      const double2 mx = q_wg_max2(in ? rv[0] : -INFINITY, in ? rv[2] : -INFINITY, red);
      const double2 sm = q_wg_sum2(in && rv[1] > 0.0 ? rv[1] * exp_nonpos((rv[0] - mx.x) * p.itemp) : 0.0,
                                   in && rv[3] > 0.0 ? rv[3] * exp_nonpos((rv[2] - mx.y) * p.itemp) : 0.0,
                                   red);
      r[0] = mx.x; r[1] = sm.x; r[2] = mx.y; r[3] = sm.y;
    } else if (kind == kQSum) {
      r[0] = q_wg_sum2(in ? rv[0] : 0.0, 0.0, red).x;
    } else {
      r[1] = q_wg_max2(in ? rv[1] : -1.0, 0.0, red).x;
      double tot;
      const double ex = q_wg_excl_scan(in ? rv[0] : 0.0, red, &tot);
      if (in) {
        xb[tid] = ex;
        xw[tid] = rv[0];
      }
      if (tid == 0) xb[G] = tot;
      r[0] = tot;
      __syncthreads();
    }
    return true;
  };

  // this chunk of node v's target and draft rows; entries outside the chunk
  // (in[e] false) load a valid address and are read as -inf by the users, so
  // the loads stay in flight until then
  bool in[kQE];
#pragma unroll
  for (int e = 0; e < kQE; ++e) in[e] = e < E && e0 + e < c1;
  auto load_rows = [&](int v, float (&lr)[kQE], float (&dr)[kQE]) __attribute__((always_inline)) {
    const float* lrow = p.tl + (size_t)v * V;
    const float* drow = p.dl + (size_t)v * V;
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      if (e < E) {                        // (uniform)
        const int yc = min(e0 + e, V - 1);
        lr[e] = lrow[yc];
        dr[e] = drow[yc];
      }
    }
  };

  double pv[kQE], qv[kQE];
  double r4[4];
  float lf[kQE], df[kQE];                 // rows of the visited node
  float pl[kQE], pd[kQE];                 // rows of its first child, fetched ahead
  int u = 0, depth = 0;
  if (lead && tid == 0) p.path[0] = 0;
  load_rows(0, lf, df);
  for (;;) {
    const float* lrow = p.tl + (size_t)u * V;
    const float* drow = p.dl + (size_t)u * V;
    const int first = fc[u];
    if (first < T) load_rows(first, pl, pd);
    // the children's logits at their tokens and their uniforms (to LDS
    // before the next barrier)
    const bool ischild = tid < T && tid > u && par[tid] == u;
    float cl = 0.f, cd = 0.f, cu = 0.f, ub = 0.f;
    if (ischild) {
      const int x = tk[tid];
      cl = lrow[x];
      cd = drow[x];
      cu = p.U[tid];
    }
    if (tid == 0) ub = p.U[T + u];
    // this chunk's row statistics
    float ml = -INFINITY, md = -INFINITY;
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      if (e < E) {                        // (uniform)
        lf[e] = in[e] ? lf[e] : -INFINITY;
        df[e] = in[e] ? df[e] : -INFINITY;
        ml = fmaxf(ml, lf[e]);
        md = fmaxf(md, df[e]);
      }
    }
    const double2 wm = q_wg_max2((double)ml, (double)md, red);
    // e^((l - m) / t) against the chunk maxima m, kept: p1 and q1 of the
    // chunk are these times one factor per row once the global maxima are known
    double sp = 0.0, sq = 0.0;
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      pv[e] = 0.0;
      qv[e] = 0.0;
      if (e < E) {                        // (uniform; -inf outside the chunk gives 0)
        pv[e] = exp_nonpos(((double)lf[e] - wm.x) * p.itemp);
        qv[e] = exp_nonpos(((double)df[e] - wm.y) * p.itemp);
        sp += pv[e];
        sq += qv[e];
      }
    }
    const double2 ws = q_wg_sum2(sp, sq, red);
    if (ischild) chu[tid] = cu;
    if (tid == 0) sh_ub = ub;
    if (!exchange(kQStats, wm.x, ws.x, wm.y, ws.y, r4)) break;
    const double M = r4[0], zp = r4[1], Md = r4[2], zq = r4[3];
    const double izp = 1.0 / zp;
    const double izq = 1.0 / zq;
    // p1 and q1 of every child at its own token, in parallel
    if (ischild) {
      cq1[tid] = exp_nonpos(((double)cd - Md) * p.itemp) * izq;
      cp1[tid] = exp_nonpos(((double)cl - M) * p.itemp) * izp;
    }
    __syncthreads();
    // children in ascending index; p_i(x), q_i(x) at x alone, replaying this
    // node's rejections; a rejection forms the residual over the vocabulary
    // (p1, q1 of this chunk scaled from the kept terms at the first one)
    int nrej = 0;
    double D = 1.0;                          // draft mass not yet rejected at u
    int next = -1;
    bool have = false, alive = true;
    for (int wd = 0; wd < kWords && next < 0 && alive; ++wd) {
      uint64_t bits = cmask[u][wd];
      while (bits != 0ull) {
        const int c = wd * 64 + __builtin_ctzll(bits);
        bits &= bits - 1ull;
        const int x = tk[c];
        bool seen = false;
        for (int r = 0; r < nrej; ++r) seen |= rej[r] == x;
        if (seen) continue;                  // a draw never repeats a token
        const double q1x = cq1[c];
        double px = cp1[c];
        for (int r = 0; r < nrej; ++r) px = fmax(px - q1x * hd[r], 0.0) * hz[r];
        const double iD = D > 0.0 ? 1.0 / D : 0.0;
        const double qx = q1x * iD;
        if ((double)chu[c] * qx < px) {
          next = c;
          break;
        }
        if (!have) {
          const double fp = exp_nonpos((wm.x - M) * p.itemp) * izp;
          const double fq = exp_nonpos((wm.y - Md) * p.itemp) * izq;
#pragma unroll
          for (int e = 0; e < kQE; ++e) {
            pv[e] *= fp;
            qv[e] *= fq;
          }
          have = true;
        }
        // rejected: p <- max(p - q, 0) / Z over the vocabulary (the same
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
          if (e0 + e == x) qv[e] = 0.0;      // x leaves q after this step's update
        const double wsum = q_wg_sum2(s, 0.0, red).x;
        if (!exchange(kQSum, wsum, 0.0, 0.0, 0.0, r4)) {
          alive = false;
          break;
        }
        const double iz = 1.0 / r4[0];
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
    }
    if (!alive) break;
    if (next >= 0) {
      ++depth;
      if (lead && tid == 0) {
        if (depth < p.max_path) p.path[depth] = next;
        else set_status(p.status, EAGLE_DEV_PATH_TRUNC);
      }
      if (next == first) {
#pragma unroll
        for (int e = 0; e < kQE; ++e) {
          lf[e] = pl[e];
          df[e] = pd[e];
        }
      } else {
        load_rows(next, lf, df);
      }
      u = next;
      __syncthreads();                       // cp1 / cq1 / chu are reused
      continue;
    }
    // bonus: the smallest token whose running sum of p exceeds U[T + u] sum(p)
    if (!have) {
      const double fp = exp_nonpos((wm.x - M) * p.itemp) * izp;
#pragma unroll
      for (int e = 0; e < kQE; ++e) pv[e] *= fp;
    }
    double own = 0.0;
    int last = -1, lastm = -1;
#pragma unroll
    for (int e = 0; e < kQE; ++e) {
      own += pv[e];
      if (pv[e] > 0.0) {
        last = e0 + e;
        lastm = e;
      }
    }
    double wtot;
    const double tpre = q_wg_excl_scan(own, red, &wtot);
    const double lastc = q_wg_max2((double)last, 0.0, red).x;
    if (!exchange(kQScan, wtot, lastc, 0.0, 0.0, r4)) break;
    const double total = r4[0];
    const int lastall = (int)r4[1];
    const double target = (double)sh_ub * total;
    // The running sums split [0, total) into consecutive intervals: chunk v
    // holds [xb[v], xb[v + 1]), thread t of it [tb[t], tb[t + 1]), and the
    // entries of a thread follow in token order.  The crossing belongs to
    // the first chunk (and in it the first thread) with mass whose interval
    // ends above target: every workgroup finds the same chunk, and only that
    // one searches.  With target >= total (rounding) it is the last token
    // with mass.
    if (target < total) {
      const bool cl = tid < G && xw[tid] > 0.0 && xb[tid + 1] > target;
      const int owner = kQT - (int)q_wg_max2(cl ? (double)(kQT - tid) : 0.0, 0.0, red).x;
      if (owner == w) {
        tb[tid] = tid == 0 ? xb[w] : fmin(xb[w] + tpre, xb[w + 1]);
        if (tid == 0) tb[kQT] = xb[w + 1];
        __syncthreads();
        const bool tc = own > 0.0 && tb[tid + 1] > target;
        const int first = kQT - (int)q_wg_max2(tc ? (double)(kQT - tid) : 0.0, 0.0, red).x;
        if (tid == first) {
          const double end = tb[tid + 1];
          double run = tb[tid];
          int hit = -1;
#pragma unroll
          for (int e = 0; e < kQE; ++e) {
            if (hit < 0 && pv[e] > 0.0) {
              const double nx = e == lastm ? end : fmin(run + pv[e], end);
              if (nx > target) hit = e0 + e;
              run = nx;
            }
          }
          p.bonus[0] = hit >= 0 ? hit : e0 + lastm;
        } else if (first >= kQT && tid == 0) {
          p.bonus[0] = max(lastall, 0);       // (no thread with mass claimed it)
        }
      } else if (owner >= kQT && lead && tid == 0) {
        p.bonus[0] = max(lastall, 0);         // (no chunk with mass claimed it)
      }
    } else if (lead && tid == 0) {
      p.bonus[0] = max(lastall, 0);
    }
    if (lead && tid == 0) {
      p.n_acc[0] = min(depth, p.max_path - 1);
      for (int d = depth + 1; d < p.max_path; ++d) p.path[d] = -1;
    }
    break;
  }
  // a new generation for the next call: its records never match this call's
  if (lead && tid == 0)
    __hip_atomic_store(p.sync, (gen + 1) & 0x1fffff, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  return 256 + (size_t)2 * eagle::kQG * 8 * sizeof(uint64_t);
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
  // 128 workgroups while they can hold the vocabulary (fewer records to
  // gather at every barrier), all CUs beyond that
  const int G = std::min(V <= eagle::kQG / 2 * eagle::kQT * eagle::kQE ? eagle::kQG / 2 : eagle::kQG,
                         q_device_cus());
  const int C = (V + G - 1) / G;
  const int E = (C + eagle::kQT - 1) / eagle::kQT;
  EAGLE_REQUIRE(E <= eagle::kQE, EAGLE_EUNSUPPORTED);
  eagle::QGridParams p{};
  p.T = T; p.V = V; p.G = G; p.C = C; p.E = E;
  p.token = node_token; p.parent = node_parent; p.tl = target_logits; p.dl = draft_logits;
  p.itemp = 1.0 / (double)temperature;
  p.U = uniforms; p.max_path = max_path; p.path = path; p.n_acc = n_accepted;
  p.bonus = bonus_token; p.status = dev_status;
  p.sync = (int32_t*)workspace;                                  // generation
  p.rec = (uint64_t*)((char*)workspace + 256);                   // [2][G][8]
  hipLaunchKernelGGL(eagle::accept_q_grid_kernel, dim3(G), dim3(eagle::kQT), 0, stream, p);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
