// KV commit after acceptance: the accepted path's K/V rows become the next
// cache positions.
//
// Sources: "Support Eagle-3 Speculative Decoding in llama.cpp", the reply on
// the draft's context - the target keeps KV only for accepted tokens and the
// draft's candidates need eviction; "EAGLE-2: Feature-Level Speculative
// Decoding Guide", Key Architectural Mechanics 3 - the accepted tokens are
// the longest verified root path.
//
// One workgroup per (KV head, K or V, layer).  The row count is read on the
// device (eagle_accept's n_accepted), so the call needs no host round trip.
// Every source row of the workgroup is loaded into LDS (16-byte loads, all of
// a thread's loads in flight before the first is used) before any cache row
// is stored, so the tree rows may sit inside the cache itself.  The count and
// the source row ids are read together, so a call waits on two dependent
// memory round trips.  The work is a
// few KB per layer: the call is bound by launch latency, not bandwidth, and
// one launch covers every layer.
#include "common.h"

namespace eagle {

constexpr int kKvThreads = 256;
constexpr int kKvStageBytes = 65536;
constexpr int kKvChunks = kKvStageBytes / 16;          // 16-byte chunks staged
constexpr int kKvPerThread = kKvChunks / kKvThreads;   // 16

struct KvParams {
  const char* src[2];      // K, V
  char* dst[2];
  int64_t src_ld, src_layer;    // bytes
  int64_t dst_ld, dst_layer;    // bytes
  int64_t head_src, head_dst;   // bytes per head block
  int64_t L;
  int src_rows, max_rows, cpr;  // cpr: 16-byte chunks per row
  const int32_t* rows;
  const int32_t* n_acc;
  int32_t* status;
};

// One (KV head, K or V, layer) of a commit.  rows: the source row ids (global
// memory, or LDS for the pair kernel), a: the accepted count minus one.
__device__ __forceinline__ void kv_commit_block(const KvParams& p, const int32_t* rows, int a,
                                                int head, int kv, int layer, u32x4* stg) {
  const int tid = threadIdx.x;
  const bool reporter = tid == 0 && head == 0 && kv == 0 && layer == 0;
  const char* src = p.src[kv] + layer * p.src_layer + head * p.head_src;
  char* dst = p.dst[kv] + layer * p.dst_layer + head * p.head_dst + p.L * p.dst_ld;
  const int total_max = p.max_rows * p.cpr;
  int r[kKvPerThread];
#pragma unroll
  for (int i = 0; i < kKvPerThread; ++i) {
    const int c = tid + kKvThreads * i;
    r[i] = c < total_max ? rows[c / p.cpr] : -1;
  }
  int n = p.max_rows;
  if (a < 0) {
    if (reporter) set_status(p.status, EAGLE_DEV_BAD_INDEX);
    n = 0;
  } else if (a + 1 > p.max_rows) {
    if (reporter) set_status(p.status, EAGLE_DEV_PATH_TRUNC);
  } else {
    n = a + 1;
  }
  const int total = n * p.cpr;
  u32x4 v[kKvPerThread];
  bool ok[kKvPerThread];
#pragma unroll
  for (int i = 0; i < kKvPerThread; ++i) {
    const int c = tid + kKvThreads * i;
    ok[i] = false;
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (c < total) {
      const int j = c / p.cpr;
      const int ch = c - j * p.cpr;
      ok[i] = r[i] >= 0 && r[i] < p.src_rows;
      if (ok[i]) v[i] = *(const u32x4*)(src + r[i] * p.src_ld + ch * 16);
      else if (ch == 0 && head == 0 && kv == 0 && layer == 0) set_status(p.status, EAGLE_DEV_BAD_INDEX);
    }
  }
#pragma unroll
  for (int i = 0; i < kKvPerThread; ++i) {
    const int c = tid + kKvThreads * i;
    if (c < total) stg[c] = v[i];
  }
  __syncthreads();  // every source row of this (layer, head) is read
#pragma unroll
  for (int i = 0; i < kKvPerThread; ++i) {
    const int c = tid + kKvThreads * i;
    if (c < total && ok[i]) {
      const int j = c / p.cpr;
      const int ch = c - j * p.cpr;
      *(u32x4*)(dst + j * p.dst_ld + ch * 16) = stg[c];
    }
  }
}

__global__ __launch_bounds__(kKvThreads) void kv_commit_kernel(KvParams p) {
  extern __shared__ u32x4 stg[];  // max_rows x cpr chunks
  // the count and this thread's source rows are read together (the rows past
  // the count are never used)
  const int a = p.n_acc ? p.n_acc[0] : p.max_rows - 1;
  kv_commit_block(p, p.rows, a, blockIdx.x, blockIdx.y, blockIdx.z, stg);
}

// The draft's rows of the accepted path: slot_of_pool[node_pool_idx[path[j]]]
// for the leading path nodes the draft expanded (every accepted node but
// possibly the last, which may be a leaf the draft never ran).  One thread per
// path entry, so the three dependent lookups are one round trip each.
struct PathSlotParams {
  const int32_t* path;
  const int32_t* n_acc;
  const int32_t* node_pool_idx;
  const int32_t* slot_of_pool;
  int32_t* rows;
  int32_t* n_rows_m1;
  int32_t* status;
  int max_path, T, pool_cap, n_slots;
};

__global__ __launch_bounds__(EAGLE_MAX_TREE) void path_slots_kernel(PathSlotParams p) {
  __shared__ int first_end;
  const int j = threadIdx.x;
  const int a = p.n_acc[0];
  if (j == 0) first_end = p.max_path;
  __syncthreads();
  const int n = a < 0 ? 0 : min(a + 1, p.max_path);
  int slot = -1;
  if (j < n) {
    const int node = p.path[j];
    bool bad = node < 0 || node >= p.T;
    if (!bad) {
      const int pi = p.node_pool_idx[node];
      bad = pi < 0 || pi >= p.pool_cap;
      if (!bad) slot = p.slot_of_pool[pi];
    }
    if (bad) set_status(p.status, EAGLE_DEV_BAD_INDEX);
    if (bad || slot < 0 || slot >= p.n_slots) atomicMin(&first_end, j);
  }
  __syncthreads();
  const int cnt = min(n, first_end);
  if (j < p.max_path) p.rows[j] = j < cnt ? slot : -1;
  if (j == 0) {
    p.n_rows_m1[0] = cnt - 1;
    if (cnt == 0) set_status(p.status, EAGLE_DEV_BAD_INDEX);
  }
}

// The draft's slot rows of the accepted path (path_slots_kernel's rule) into
// LDS rows[], one thread per path entry; returns the row count minus one.
__device__ __forceinline__ int path_slot_rows(const PathSlotParams& p, int32_t* rows,
                                              int* first_end) {
  const int j = threadIdx.x;
  const int a = p.n_acc[0];
  if (j == 0) *first_end = p.max_path;
  __syncthreads();
  const int n = a < 0 ? 0 : min(a + 1, p.max_path);
  int slot = -1;
  if (j < n) {
    const int node = p.path[j];
    bool bad = node < 0 || node >= p.T;
    if (!bad) {
      const int pi = p.node_pool_idx[node];
      bad = pi < 0 || pi >= p.pool_cap;
      if (!bad) slot = p.slot_of_pool[pi];
    }
    if (bad) set_status(p.status, EAGLE_DEV_BAD_INDEX);
    if (bad || slot < 0 || slot >= p.n_slots) atomicMin(first_end, j);
  }
  __syncthreads();
  const int cnt = min(n, *first_end);
  if (j < p.max_path) rows[j] = j < cnt ? slot : -1;
  if (cnt == 0 && j == 0) set_status(p.status, EAGLE_DEV_BAD_INDEX);
  __syncthreads();
  return cnt - 1;
}

// Both commits of a cycle in one launch: blockIdx.z = 0 appends the target's
// accepted rows (tgt, rows = the path), blockIdx.z = 1 the draft's rows of
// the same nodes (drf, rows found from the path as by eagle_path_slots).
__global__ __launch_bounds__(kKvThreads) void kv_commit_pair_kernel(KvParams tgt, KvParams drf,
                                                                    PathSlotParams ps) {
  extern __shared__ u32x4 stg[];
  __shared__ int32_t srows[EAGLE_MAX_TREE];
  __shared__ int first_end;
  if (blockIdx.z == 0) {
    const int a = tgt.n_acc[0];
    kv_commit_block(tgt, tgt.rows, a, blockIdx.x, blockIdx.y, 0, stg);
  } else {
    const int a = path_slot_rows(ps, srows, &first_end);
    kv_commit_block(drf, srows, a, blockIdx.x, blockIdx.y, 0, stg);
  }
}

}  // namespace eagle

extern "C" int eagle_kv_commit(const void* src_k, const void* src_v, int32_t ld_src,
                               int32_t src_rows, int64_t src_layer_stride, const int32_t* rows,
                               const int32_t* n_accepted, int32_t max_rows, void* cache_k,
                               void* cache_v, int64_t L, int64_t ld_cache,
                               int64_t cache_layer_stride, int32_t layers, int32_t Hkv,
                               int32_t hd, eagle_dtype dt, int32_t* dev_status,
                               hipStream_t stream) {
  using namespace eagle;
  EAGLE_REQUIRE(src_k && src_v && rows && cache_k && cache_v, EAGLE_EINVAL);
  EAGLE_REQUIRE(dt == EAGLE_BF16 || dt == EAGLE_F32, EAGLE_EINVAL);
  EAGLE_REQUIRE(Hkv >= 1 && layers >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(max_rows >= 1 && max_rows <= EAGLE_MAX_TREE, EAGLE_EINVAL);
  EAGLE_REQUIRE(src_rows >= 1 && src_rows <= ld_src, EAGLE_EINVAL);
  EAGLE_REQUIRE(L >= 0 && ld_cache >= 1 && L + max_rows <= ld_cache, EAGLE_EINVAL);
  EAGLE_REQUIRE(hd == 64 || hd == 128, EAGLE_EUNSUPPORTED);
  const int64_t es = dt == EAGLE_BF16 ? 2 : 4;
  EAGLE_REQUIRE((int64_t)max_rows * hd * es <= kKvStageBytes, EAGLE_EUNSUPPORTED);
  const int64_t src_layer = (int64_t)Hkv * ld_src * hd;
  const int64_t dst_layer = (int64_t)Hkv * ld_cache * hd;
  EAGLE_REQUIRE(layers == 1 || (src_layer_stride >= src_layer && cache_layer_stride >= dst_layer),
                EAGLE_EINVAL);
  const uintptr_t al = (uintptr_t)src_k | (uintptr_t)src_v | (uintptr_t)cache_k |
                       (uintptr_t)cache_v;
  EAGLE_REQUIRE((al & 15) == 0, EAGLE_EINVAL);
  KvParams p{};
  p.src[0] = (const char*)src_k;
  p.src[1] = (const char*)src_v;
  p.dst[0] = (char*)cache_k;
  p.dst[1] = (char*)cache_v;
  p.src_ld = (int64_t)hd * es;
  p.dst_ld = (int64_t)hd * es;
  p.head_src = (int64_t)ld_src * hd * es;
  p.head_dst = ld_cache * hd * es;
  p.src_layer = (layers == 1 ? src_layer : src_layer_stride) * es;
  p.dst_layer = (layers == 1 ? dst_layer : cache_layer_stride) * es;
  p.L = L;
  p.src_rows = src_rows;
  p.max_rows = max_rows;
  p.cpr = (int)(hd * es / 16);
  p.rows = rows;
  p.n_acc = n_accepted;
  p.status = dev_status;
  hipLaunchKernelGGL(kv_commit_kernel, dim3(Hkv, 2, layers), dim3(kKvThreads),
                     (size_t)max_rows * hd * es, stream, p);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_path_slots(const int32_t* path, const int32_t* n_accepted, int32_t max_path,
                                const int32_t* node_pool_idx, int32_t T,
                                const int32_t* slot_of_pool, int32_t pool_cap, int32_t n_slots,
                                int32_t* slot_rows, int32_t* n_rows_minus_one,
                                int32_t* dev_status, hipStream_t stream) {
  using namespace eagle;
  EAGLE_REQUIRE(path && n_accepted && node_pool_idx && slot_of_pool && slot_rows &&
                    n_rows_minus_one, EAGLE_EINVAL);
  EAGLE_REQUIRE(max_path >= 1 && max_path <= EAGLE_MAX_TREE, EAGLE_EINVAL);
  EAGLE_REQUIRE(T >= 1 && T <= EAGLE_MAX_TREE && pool_cap >= 1 && n_slots >= 1, EAGLE_EINVAL);
  PathSlotParams p{path, n_accepted, node_pool_idx, slot_of_pool, slot_rows, n_rows_minus_one,
                   dev_status, max_path, T, pool_cap, n_slots};
  hipLaunchKernelGGL(path_slots_kernel, dim3(1), dim3(EAGLE_MAX_TREE), 0, stream, p);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_kv_commit_pair(
    const void* t_src_k, const void* t_src_v, int32_t t_ld_src, int32_t t_src_rows,
    void* t_cache_k, void* t_cache_v, int64_t t_ld_cache, const void* d_src_k,
    const void* d_src_v, int32_t d_ld_src, int32_t d_src_rows, void* d_cache_k, void* d_cache_v,
    int64_t d_ld_cache, int64_t L, const int32_t* path, const int32_t* n_accepted,
    int32_t max_rows, const int32_t* node_pool_idx, int32_t T, const int32_t* slot_of_pool,
    int32_t pool_cap, int32_t max_path, int32_t Hkv, int32_t hd, eagle_dtype dt,
    int32_t* dev_status, hipStream_t stream) {
  using namespace eagle;
  EAGLE_REQUIRE(t_src_k && t_src_v && t_cache_k && t_cache_v && d_src_k && d_src_v && d_cache_k &&
                    d_cache_v && path && n_accepted && node_pool_idx && slot_of_pool,
                EAGLE_EINVAL);
  EAGLE_REQUIRE(dt == EAGLE_BF16 || dt == EAGLE_F32, EAGLE_EINVAL);
  EAGLE_REQUIRE(Hkv >= 1 && hd >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(hd == 64 || hd == 128, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(max_rows >= 1 && max_rows <= EAGLE_MAX_TREE && max_path >= 1 &&
                    max_path <= max_rows, EAGLE_EINVAL);
  EAGLE_REQUIRE(t_src_rows >= 1 && t_src_rows <= t_ld_src && d_src_rows >= 1 &&
                    d_src_rows <= d_ld_src, EAGLE_EINVAL);
  EAGLE_REQUIRE(L >= 0 && L + max_rows <= t_ld_cache && L + max_path <= d_ld_cache, EAGLE_EINVAL);
  EAGLE_REQUIRE(T >= 1 && T <= EAGLE_MAX_TREE && pool_cap >= 1, EAGLE_EINVAL);
  const int64_t es = dt == EAGLE_BF16 ? 2 : 4;
  EAGLE_REQUIRE((int64_t)max_rows * hd * es <= kKvStageBytes, EAGLE_EUNSUPPORTED);
  const uintptr_t al = (uintptr_t)t_src_k | (uintptr_t)t_src_v | (uintptr_t)t_cache_k |
                       (uintptr_t)t_cache_v | (uintptr_t)d_src_k | (uintptr_t)d_src_v |
                       (uintptr_t)d_cache_k | (uintptr_t)d_cache_v;
  EAGLE_REQUIRE((al & 15) == 0, EAGLE_EINVAL);
  auto desc = [&](const void* sk, const void* sv, int32_t ld_src, int32_t src_rows, void* ck,
                  void* cv, int64_t ld_cache, int32_t rows_max) {
    KvParams p{};
    p.src[0] = (const char*)sk;
    p.src[1] = (const char*)sv;
    p.dst[0] = (char*)ck;
    p.dst[1] = (char*)cv;
    p.src_ld = (int64_t)hd * es;
    p.dst_ld = (int64_t)hd * es;
    p.head_src = (int64_t)ld_src * hd * es;
    p.head_dst = ld_cache * hd * es;
    p.src_layer = 0;
    p.dst_layer = 0;
    p.L = L;
    p.src_rows = src_rows;
    p.max_rows = rows_max;
    p.cpr = (int)(hd * es / 16);
    p.n_acc = n_accepted;
    p.status = dev_status;
    return p;
  };
  KvParams tgt = desc(t_src_k, t_src_v, t_ld_src, t_src_rows, t_cache_k, t_cache_v, t_ld_cache,
                      max_rows);
  tgt.rows = path;
  KvParams drf = desc(d_src_k, d_src_v, d_ld_src, d_src_rows, d_cache_k, d_cache_v, d_ld_cache,
                      max_path);
  drf.rows = nullptr;   // found in the kernel
  PathSlotParams ps{path, n_accepted, node_pool_idx, slot_of_pool, nullptr, nullptr,
                    dev_status, max_path, T, pool_cap, d_src_rows};
  hipLaunchKernelGGL(kv_commit_pair_kernel, dim3(Hkv, 2, 2), dim3(kKvThreads),
                     (size_t)max_rows * hd * es, stream, tgt, drf, ps);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
