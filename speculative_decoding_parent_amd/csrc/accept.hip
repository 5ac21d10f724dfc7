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
// replacement).  A prepass over all rows (accept_row_stats_kernel, many
// workgroups) gives each row's chunk (max, sum); then one workgroup walks
// the tree.  At a node the row normalisers Zp, Zq come from the chunk
// statistics and child i with token x is accepted iff U[c] (q(x) / Zq) <
// p(x) / Zp, with p = e^((l - max l) / t), q = e^((d - max d) / t) evaluated
// for x alone.  Only a rejection (or the bonus draw) writes the node's
// unnormalised rows into the workspace (pres, qres); a rejection then turns
// pres into max(pres / Zp - qres / Zq, 0) (one pass over the vocabulary,
// with the reciprocals of Zp and Zq),
// drops x from qres and Zq, and the next child is tried.  The bonus is drawn
// from the last pres by inverse CDF.  Sums are taken in a fixed order (each
// thread's elements in index order, then a fixed butterfly, then the waves in
// order), so the result does not depend on timing.
constexpr int kQThreads = 1024;
constexpr int kQWaves = kQThreads / 64;
constexpr int kQBatch = 8;

__device__ __forceinline__ double q_block_sum(double v, double* dred) {
  v = wave_sum_d(v);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) dred[tid >> 6] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < kQWaves; ++w) s += dred[w];
  return s;
}

__device__ __forceinline__ float q_block_max(float v, float* fred) {
  v = wave_max(v);
  const int tid = threadIdx.x;
  __syncthreads();
  if ((tid & 63) == 0) fred[tid >> 6] = v;
  __syncthreads();
  float m = -INFINITY;
  for (int w = 0; w < kQWaves; ++w) m = fmaxf(m, fred[w]);
  return m;
}

__global__ __launch_bounds__(kQThreads) void accept_sample_q_kernel(
    int T, const int32_t* __restrict__ token, const int32_t* __restrict__ parent,
    const float* __restrict__ tl, const float* __restrict__ dl, int V, double itemp,
    const float* __restrict__ U, const double* __restrict__ pst, const double* __restrict__ qst,
    int nchunk, double* pres, double* qres, int max_path,
    int32_t* __restrict__ path, int32_t* __restrict__ n_acc, int32_t* __restrict__ bonus,
    int32_t* __restrict__ status) {
  __shared__ int32_t par[EAGLE_MAX_TREE];
  __shared__ int32_t tk[EAGLE_MAX_TREE];
  __shared__ int32_t kid[EAGLE_MAX_TREE];
  __shared__ int32_t rej[EAGLE_MAX_TREE];
  __shared__ double dred[kQWaves];
  __shared__ float fred[kQWaves];
  __shared__ double csum[kQThreads];
  __shared__ int sh_nk, sh_hit, sh_acc;
  __shared__ double sh_qx, sh_ml, sh_md, sh_zp, sh_zq;
  const int tid = threadIdx.x;
  for (int i = tid; i < T; i += kQThreads) {
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
  __syncthreads();
  int u = 0, depth = 0;
  if (tid == 0) path[0] = 0;
  for (;;) {
    const float* lrow = tl + (size_t)u * V;
    const float* drow = dl + (size_t)u * V;
    // the row's max and normaliser from the prepass's chunk statistics
    // (combined in chunk order by wave 0); p(x) and q(x) of single tokens
    // from the logits; the rows are written out over the vocabulary only
    // when a rejection or the bonus draw needs them
    if (tid < 64) {
      double a = -INFINITY, b = -INFINITY;
      for (int c = tid; c < nchunk; c += 64) {
        a = fmax(a, pst[((size_t)u * nchunk + c) * 2]);
        b = fmax(b, qst[((size_t)u * nchunk + c) * 2]);
      }
      a = wave_max_d(a);
      b = wave_max_d(b);
      double za = 0.0, zb = 0.0;
      for (int c = tid; c < nchunk; c += 64) {
        const double* x = pst + ((size_t)u * nchunk + c) * 2;
        const double* y = qst + ((size_t)u * nchunk + c) * 2;
        za += x[1] * exp_nonpos((x[0] - a) * itemp);
        zb += y[1] * exp_nonpos((y[0] - b) * itemp);
      }
      za = wave_sum_d(za);
      zb = wave_sum_d(zb);
      if (tid == 0) {
        sh_ml = a;
        sh_md = b;
        sh_zp = za;
        sh_zq = zb;
      }
    }
    __syncthreads();
    const double ml = sh_ml, md = sh_md;
    double zp = sh_zp, zq = sh_zq;
    bool rows_out = false;   // pres / qres hold this node's rows
    // writes pres = p (unnormalised) and qres = q over the vocabulary
    auto rows = [&]() __attribute__((always_inline)) {
      for (int v0 = tid; v0 < V; v0 += kQThreads * kQBatch) {
        float a[kQBatch], b[kQBatch];
#pragma unroll
        for (int i = 0; i < kQBatch; ++i) {
          const int v = v0 + i * kQThreads;
          a[i] = v < V ? lrow[v] : 0.f;
          b[i] = v < V ? drow[v] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kQBatch; ++i) {
          const int v = v0 + i * kQThreads;
          if (v < V) {
            pres[v] = exp_nonpos(((double)a[i] - ml) * itemp);
            qres[v] = exp_nonpos(((double)b[i] - md) * itemp);
          }
        }
      }
      rows_out = true;
    };
    if (tid == 0) {
      int n = 0;
      for (int c = u + 1; c < T; ++c)
        if (par[c] == u) kid[n++] = c;
      sh_nk = n;
    }
    __syncthreads();
    const int nk = sh_nk;
    int nrej = 0;
    int next = -1;
    for (int i = 0; i < nk; ++i) {
      const int c = kid[i];
      const int x = tk[c];
      bool seen = false;
      for (int r = 0; r < nrej; ++r) seen |= rej[r] == x;
      if (seen) continue;                 // a draw never repeats a token
      // thread 0 decides and shares the decision and q(x), so every thread
      // takes the same branch (the rejection pass below has barriers)
      if (tid == 0) {
        const double qx = rows_out ? qres[x] : exp_nonpos(((double)drow[x] - md) * itemp);
        const double px = rows_out ? pres[x] : exp_nonpos(((double)lrow[x] - ml) * itemp);
        const double qn = zq > 0.0 ? qx / zq : 0.0;   // (no draft mass left: q counts as 0)
        sh_acc = (double)U[c] * qn < px / zp;
        sh_qx = qx;
      }
      __syncthreads();
      const double qx = sh_qx;
      if (sh_acc) {
        next = c;
        break;
      }
      // rejected: p <- max(p / Zp - q / Zq, 0), q <- q without x
      if (!rows_out) {
        rows();
        __syncthreads();
      }
      double s = 0.0;
      const double izp = 1.0 / zp;
      const double izq = zq > 0.0 ? 1.0 / zq : 0.0;
      for (int v0 = tid; v0 < V; v0 += kQThreads * kQBatch) {
        double a[kQBatch], b[kQBatch];
#pragma unroll
        for (int i = 0; i < kQBatch; ++i) {
          const int v = v0 + i * kQThreads;
          a[i] = v < V ? pres[v] : 0.0;
          b[i] = v < V ? qres[v] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < kQBatch; ++i) {
          const int v = v0 + i * kQThreads;
          if (v < V) {
            const double r = fmax(a[i] * izp - b[i] * izq, 0.0);
            pres[v] = r;
            s += r;
          }
        }
      }
      zp = q_block_sum(s, dred);        // (its barriers also order the pres stores)
      if (tid == 0) {
        qres[x] = 0.0;
        rej[nrej] = x;
      }
      zq = zq - qx;
      ++nrej;
      __syncthreads();
    }
    if (next >= 0) {
      ++depth;
      if (tid == 0) {
        if (depth < max_path) path[depth] = next;
        else set_status(status, EAGLE_DEV_PATH_TRUNC);
      }
      u = next;
      __syncthreads();
      continue;
    }
    // bonus: smallest token whose running sum of pres exceeds U[T + u] Zp.
    // Thread t owns the contiguous tokens [t C, (t + 1) C).
    if (!rows_out) {
      rows();
      __syncthreads();
    }
    const double target = (double)U[T + u] * zp;
    const int C = (V + kQThreads - 1) / kQThreads;
    const int v0 = tid * C;
    const int v1 = min(V, v0 + C);
    double own = 0.0;
    for (int w0 = v0; w0 < v1; w0 += kQBatch) {
      double a[kQBatch];
#pragma unroll
      for (int i = 0; i < kQBatch; ++i) a[i] = w0 + i < v1 ? pres[w0 + i] : 0.0;
#pragma unroll
      for (int i = 0; i < kQBatch; ++i) own += a[i];
    }
    csum[tid] = own;
    if (tid == 0) sh_hit = 0x7fffffff;
    __syncthreads();
    if (tid == 0) {
      double run = 0.0;
      for (int t = 0; t < kQThreads; ++t) {
        const double nx = run + csum[t];
        csum[t] = run;                    // exclusive prefix
        run = nx;
      }
    }
    __syncthreads();
    {
      // the crossing: one token in exact arithmetic; rounding at a chunk
      // border can show it to two threads, and the lower token wins
      double run = csum[tid];
      bool found = false;
      for (int w0 = v0; w0 < v1 && !found; w0 += kQBatch) {
        double a[kQBatch];
#pragma unroll
        for (int i = 0; i < kQBatch; ++i) a[i] = w0 + i < v1 ? pres[w0 + i] : 0.0;
#pragma unroll
        for (int i = 0; i < kQBatch; ++i) {
          const int v = w0 + i;
          const double nx = run + a[i];
          if (!found && v < v1 && run <= target && nx > target) {
            atomicMin(&sh_hit, v);
            found = true;
          }
          run = nx;
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      int b = sh_hit == 0x7fffffff ? -1 : sh_hit;
      if (b < 0) {                        // rounding left none: the last token with mass
        for (int v = V - 1; v >= 0; --v)
          if (pres[v] > 0.0) {
            b = v;
            break;
          }
        b = max(b, 0);
      }
      bonus[0] = b;
      n_acc[0] = depth;
      for (int d = depth + 1; d < max_path; ++d) path[d] = -1;
    }
    return;
  }
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

extern "C" size_t eagle_accept_q_workspace(int32_t T, int32_t V) {
  if (T < 1 || V < 1) return 0;
  return (size_t)2 * (size_t)V * sizeof(double) + 2 * eagle_accept_workspace(T, V);
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
  EAGLE_REQUIRE(workspace && ((uintptr_t)workspace & 7) == 0, EAGLE_EINVAL);
  EAGLE_REQUIRE(ws_bytes >= eagle_accept_q_workspace(T, V), EAGLE_EWORKSPACE);
  const int nchunk = (V + eagle::kAcceptChunk - 1) / eagle::kAcceptChunk;
  const double itemp = 1.0 / (double)temperature;
  double* pres = (double*)workspace;
  double* pst = pres + 2 * (size_t)V;
  double* qst = pst + (size_t)T * nchunk * 2;
  hipLaunchKernelGGL(eagle::accept_row_stats_kernel, dim3(nchunk, 2 * T), dim3(256), 0, stream,
                     target_logits, pst, T, draft_logits, qst, V, itemp, nchunk);
  EAGLE_LAUNCH_CHECK();
  hipLaunchKernelGGL(eagle::accept_sample_q_kernel, dim3(1), dim3(eagle::kQThreads), 0, stream, T,
                     node_token, node_parent, target_logits, draft_logits, V, itemp, uniforms,
                     pst, qst, nchunk, pres, pres + V, max_path, path, n_accepted, bonus_token,
                     dev_status);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
