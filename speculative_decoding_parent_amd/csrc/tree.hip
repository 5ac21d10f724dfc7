// Dynamic draft tree: EXPAND (grow by cumulative log-probability) and RERANK
// (prune to the T best nodes).
//
// Sources: "Support Eagle-3 Speculative Decoding in llama.cpp" - confidence
// approximates acceptance, the tree is grown from it and pruned at the end of
// drafting; "EAGLE-2: Feature-Level Speculative Decoding Guide", section 2 -
// the token budget goes where confidence is high.  Reading: value = fp32 sum
// of log-probabilities along the root path, ties to the lower pool index.
//
// Both modes fit one workgroup (<= 4096 appended entries, <= 8192 pool
// entries).  Selection follows (value desc, index asc), a total order, so the
// result does not depend on thread scheduling: EXPAND keeps an entry when
// fewer than k_select entries beat it; RERANK sorts the pool's selection keys
// (the same order as one 64-bit number, NaN last) with a bitonic network and
// keeps the root and the first T-1 other entries.  Values are single IEEE
// fp32 adds (__fadd_rn), never contracted.
#include "common.h"

namespace eagle {

__global__ __launch_bounds__(1024) void expand_kernel(
    int32_t* __restrict__ tok, int32_t* __restrict__ par, int32_t* __restrict__ dep,
    float* __restrict__ val, int pool_n, const int32_t* __restrict__ frontier, int kf,
    const int32_t* __restrict__ cid, const float* __restrict__ clogp, int k, int ksel,
    int32_t* __restrict__ new_frontier, int32_t* __restrict__ status) {
  __shared__ float vs[EAGLE_MAX_APPEND];
  __shared__ uint8_t sel[EAGLE_MAX_APPEND];
  const int n = kf * k;
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    const int s = t / k;
    int u = frontier[s];
    if (u < 0 || u >= pool_n) {
      set_status(status, EAGLE_DEV_BAD_INDEX);
      u = 0;
    }
    const float v = __fadd_rn(val[u], clogp[t]);
    const int e = pool_n + t;
    tok[e] = cid[t];
    par[e] = u;
    dep[e] = dep[u] + 1;
    val[e] = v;
    vs[t] = v;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    const float v = vs[t];
    int rank = 0;
    for (int o = 0; o < n; ++o) rank += better(vs[o], o, v, t) ? 1 : 0;
    sel[t] = rank < ksel ? 1 : 0;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    if (!sel[t]) continue;
    int pos = 0;
    for (int o = 0; o < t; ++o) pos += sel[o];
    // exactly k_select entries rank below k_select unless values are NaN
    if (pos < ksel) new_frontier[pos] = pool_n + t;
  }
}

__global__ __launch_bounds__(1024) void rerank_kernel(
    const int32_t* __restrict__ tok, const int32_t* __restrict__ par,
    const int32_t* __restrict__ dep, const float* __restrict__ val, int pool_n, int T,
    int32_t* __restrict__ node_token, int32_t* __restrict__ node_parent,
    int32_t* __restrict__ node_depth, int32_t* __restrict__ node_pool_idx,
    int32_t* __restrict__ status) {
  __shared__ selkey_t ks[EAGLE_MAX_POOL];
  __shared__ int16_t pos[EAGLE_MAX_POOL];
  __shared__ int32_t cnt[1024];
  __shared__ int root_at;
  const int tid = threadIdx.x;
  // Selection keys (value desc, then index asc, as one number; key 0 pads
  // the power-of-two length), bitonic-sorted into descending order.
  int N = 2;
  while (N < pool_n) N <<= 1;
  for (int i = tid; i < N; i += blockDim.x) {
    ks[i] = i < pool_n ? sel_key(val[i], i) : 0ull;
    if (i < pool_n) pos[i] = 0;
  }
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int c = tid; c < N / 2; c += blockDim.x) {
        const int a = 2 * c - (c & (stride - 1));  // partner a + stride
        const bool down = (a & size) == 0;          // this run sorts descending
        const selkey_t x = ks[a], y = ks[a + stride];
        if (down ? x < y : x > y) {
          ks[a] = y;
          ks[a + stride] = x;
        }
      }
      __syncthreads();
    }
  }
  // keep: the root always, and the first T-1 non-root entries of the order
  for (int q = tid; q < pool_n; q += blockDim.x)
    if (key_index(ks[q]) == 0) root_at = q;
  __syncthreads();
  const int r0 = root_at;
  for (int q = tid; q < T; q += blockDim.x) {
    const int i = key_index(ks[q]);
    if (i == 0 || q < T - 1 || r0 < q) pos[i] = 1;
  }
  if (tid == 0 && r0 >= T) pos[0] = 1;
  __syncthreads();
  const int per = (pool_n + blockDim.x - 1) / blockDim.x;
  const int lo = tid * per;
  const int hi = min(pool_n, lo + per);
  int mine = 0;
  for (int i = lo; i < hi; ++i) mine += pos[i];
  // exclusive scan of the per-thread counts: within each wave, then over the
  // wave totals
  int incl = mine;
  const int lane = tid & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) cnt[tid >> 6] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < (tid >> 6); ++w) off += cnt[w];
  int run = off + incl - mine;
  for (int i = lo; i < hi; ++i) {
    if (pos[i]) {
      pos[i] = (int16_t)run;
      ++run;
    } else {
      pos[i] = -1;
    }
  }
  __syncthreads();
  for (int i = tid; i < pool_n; i += blockDim.x) {
    const int p = pos[i];
    if (p < 0 || p >= T) continue;
    node_token[p] = tok[i];
    node_depth[p] = dep[i];
    node_pool_idx[p] = i;
    const int pp = par[i];
    int np = -1;
    if (pp != -1) {
      if (pp < 0 || pp >= i) {
        set_status(status, EAGLE_DEV_BAD_PARENT);
      } else if (pos[pp] < 0) {
        set_status(status, EAGLE_DEV_ORPHAN);
      } else {
        np = pos[pp];
      }
    }
    node_parent[p] = np;
  }
}

// Confidence gate: one thread per drafted node.  Child j is kept while fewer
// than max_branch are kept and logp_j - logp_0 >= -ln(tau) (one fp32
// subtraction and compare, as written); the rest become -inf.
__global__ __launch_bounds__(64) void gate_children_kernel(const float* __restrict__ lp, int rows,
                                                           int k, float neg_ln_tau,
                                                           int max_branch, float* out,
                                                           int32_t* kept, float* conf) {
  const int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= rows) return;
  const float* x = lp + (size_t)r * k;
  float* y = out + (size_t)r * k;
  const float l0 = x[0];
  const float l1 = k > 1 ? x[1] : 0.f;
  int n = 0;
  for (int j = 0; j < k; ++j) {
    const float v = x[j];
    const bool keep = (n < max_branch) & (__fsub_rn(v, l0) >= neg_ln_tau);
    n += keep ? 1 : 0;
    y[j] = keep ? v : -INFINITY;
  }
  if (kept) kept[r] = n;
  if (conf) conf[r] = k > 1 ? expf(__fsub_rn(l0, l1)) : INFINITY;
}

}  // namespace eagle

extern "C" int eagle_expand_rerank(int32_t mode, int32_t* pool_token, int32_t* pool_parent,
                                   int32_t* pool_depth, float* pool_value, int32_t pool_n,
                                   int32_t pool_cap, const int32_t* frontier, int32_t kf,
                                   const int32_t* child_id, const float* child_logp, int32_t k,
                                   int32_t k_select, int32_t* new_frontier, int32_t T,
                                   int32_t* node_token, int32_t* node_parent,
                                   int32_t* node_depth, int32_t* node_pool_idx,
                                   int32_t* dev_status, hipStream_t stream) {
  EAGLE_REQUIRE(pool_token && pool_parent && pool_depth && pool_value, EAGLE_EINVAL);
  EAGLE_REQUIRE(pool_n >= 1 && pool_n <= pool_cap, EAGLE_EINVAL);
  if (mode == EAGLE_EXPAND) {
    EAGLE_REQUIRE(frontier && child_id && child_logp && new_frontier, EAGLE_EINVAL);
    EAGLE_REQUIRE(kf >= 1 && k >= 1, EAGLE_EINVAL);
    EAGLE_REQUIRE((int64_t)kf * k <= EAGLE_MAX_APPEND, EAGLE_EINVAL);
    EAGLE_REQUIRE((int64_t)pool_n + (int64_t)kf * k <= pool_cap, EAGLE_EINVAL);
    EAGLE_REQUIRE(k_select >= 1 && k_select <= kf * k, EAGLE_EINVAL);
    hipLaunchKernelGGL(eagle::expand_kernel, dim3(1), dim3(1024), 0, stream, pool_token,
                       pool_parent, pool_depth, pool_value, pool_n, frontier, kf, child_id,
                       child_logp, k, k_select, new_frontier, dev_status);
  } else if (mode == EAGLE_RERANK) {
    EAGLE_REQUIRE(node_token && node_parent && node_depth && node_pool_idx, EAGLE_EINVAL);
    EAGLE_REQUIRE(pool_n <= EAGLE_MAX_POOL, EAGLE_EINVAL);
    EAGLE_REQUIRE(T >= 1 && T <= pool_n && T <= EAGLE_MAX_TREE, EAGLE_EINVAL);
    hipLaunchKernelGGL(eagle::rerank_kernel, dim3(1), dim3(1024), 0, stream, pool_token,
                       pool_parent, pool_depth, pool_value, pool_n, T, node_token, node_parent,
                       node_depth, node_pool_idx, dev_status);
  } else {
    return EAGLE_EINVAL;
  }
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_gate_children(const float* logp, int32_t rows, int32_t k, float tau,
                                   int32_t max_branch, float* out_logp, int32_t* kept,
                                   float* confidence, hipStream_t stream) {
  using namespace eagle;
  EAGLE_REQUIRE(logp && out_logp, EAGLE_EINVAL);
  EAGLE_REQUIRE(rows >= 1 && k >= 1 && k <= EAGLE_MAX_TOPK && max_branch >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(tau >= 1.0f && tau < INFINITY, EAGLE_EINVAL);
  const float neg_ln_tau = (float)(-log((double)tau));
  hipLaunchKernelGGL(gate_children_kernel, dim3((rows + 63) / 64), dim3(64), 0, stream, logp, rows,
                     k, neg_ln_tau, max_branch, out_logp, kept, confidence);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
