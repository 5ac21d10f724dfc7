// LM head, softmax statistics and top-k.
//
// Sources: "EAGLE-2: Feature-Level Speculative Decoding Guide", Key
// Architectural Mechanics 1 - P = softmax(W_LM f) through the target's own LM
// head; section 2 - the confidence ratio of the two most likely tokens;
// "Support Eagle-3 Speculative Decoding in llama.cpp" printout - no bias.
//
// bf16 path (the hot one).  logits[t][v] = sum_k f[t][k] W[v][k] with T <= 256
// feature rows and V up to ~152K vocabulary rows of d <= 8192: at T <= 128 the
// work is ~T flop per weight byte, so the kernel is bound by streaming W from
// HBM once.  Design:
//   * MFMA v_mfma_f32_16x16x32_bf16 with W rows as the M dimension (16 rows per
//     tile, 8 or 4 tiles = 128 or 64 rows per wave, 4 waves per workgroup) and the
//     feature rows as N (16 per tile, NT tiles).  W goes straight from HBM into
//     MFMA A operands (the shared weight-streaming core, wstream.h).
//   * f is shared by all workgroups (<= 512 KB at T = 64): each 128-wide k
//     slice is staged once per workgroup in LDS (double-buffered, rows padded
//     by 16 bytes so the 16 lanes of a b128 read hit distinct banks).
//   * W for step k+1 is requested before the MFMAs of step k run.
//   * Epilogue, per wave and feature row: the 64 logits are reduced to
//     (max, sum exp(l - max)) and to the wave's top-k by (logit desc,
//     index asc); optional fp32 logits are written with 16-byte stores.
//   * A second kernel merges the per-wave partials of each row in a fixed
//     order: lse = M + log(sum s_w exp(m_w - M)); for the top-k it keeps only
//     the list prefixes that can still reach the top k and selects among them.
// fp32 path (small workloads): a plain VALU dot product per logit, then a
// per-row top-k kernel.
#include "wstream.h"

namespace eagle {

constexpr int kLmWaves = 4;

// W tiles of 16 rows per wave: 8 (128 rows) while the feature rows fit one MFMA
// tile, which keeps the most weight bytes in flight per wave; fewer as more
// feature rows need accumulator registers (no spills up to T = 256).
__host__ __device__ constexpr int lm_mt(int T) {
  return T <= 16 ? 8 : (T <= 128 ? 2 : 1);
}

struct LmParams {
  const bf16_t* f;
  const bf16_t* W;
  int T, d, V, k;
  float* logits;
  float2* part_stat;   // [nwave][T]
  float* part_val;     // [nwave][T][k]
  int32_t* part_idx;   // [nwave][T][k]
};

template <int NT, int kLmMT>
__global__ __launch_bounds__(256, (kLmMT >= 8 || NT >= 16 ? 1 : 2)) void lmhead_bf16_kernel(
    LmParams p) {
  constexpr int kLmRowsWave = 16 * kLmMT;
  constexpr int kLmRowsBlock = kLmRowsWave * kLmWaves;
  __shared__ __attribute__((aligned(16))) bf16_t fs[ws_lds_elems<NT>()];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int v0 = blockIdx.x * kLmRowsBlock + wave * kLmRowsWave;

  const bf16_t* wrow[kLmMT];
#pragma unroll
  for (int mt = 0; mt < kLmMT; ++mt) {
    const int v = min(v0 + mt * 16 + r16, p.V - 1);
    wrow[mt] = p.W + (size_t)v * p.d + g * 8;
  }
  f32x4 acc[kLmMT][NT];
  wstream_mfma<NT, kLmMT>(wrow, p.f, p.d, p.T, p.d, fs, acc);

  // ---- epilogue.  Lane (g, r16) holds, for tile (mt, nt), the logits of
  // vocabulary rows v0 + 16 mt + 4 g + j (j < 4) for feature row 16 nt + r16.
  const int T = p.T;
  const int V = p.V;
  const int wglob = blockIdx.x * kLmWaves + wave;
  if (p.logits) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int t = nt * 16 + r16;
      if (t >= T) continue;
      float* out = p.logits + (size_t)t * V;
#pragma unroll
      for (int mt = 0; mt < kLmMT; ++mt) {
        const int vb = v0 + mt * 16 + 4 * g;
        if ((V & 3) == 0 && vb + 3 < V) {
          *(f32x4*)(out + vb) = acc[mt][nt];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (vb + j < V) out[vb + j] = acc[mt][nt][j];
        }
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = nt * 16 + r16;
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < kLmMT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v0 + mt * 16 + 4 * g + j < V) m = fmaxf(m, acc[mt][nt][j]);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    float s = 0.f;
#pragma unroll
    for (int mt = 0; mt < kLmMT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v0 + mt * 16 + 4 * g + j < V) s += expf(acc[mt][nt][j] - m);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (g == 0 && t < T) p.part_stat[(size_t)wglob * T + t] = make_float2(m, s);

    // wave top-k of this feature row: k rounds of "best not yet taken"
    uint32_t taken = 0;
    for (int r = 0; r < p.k; ++r) {
      float bv = -INFINITY;
      int bi = INT_MAX;
#pragma unroll
      for (int mt = 0; mt < kLmMT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = v0 + mt * 16 + 4 * g + j;
          const float x = acc[mt][nt][j];
          if (v < V && !((taken >> (mt * 4 + j)) & 1u) && better(x, v, bv, bi)) {
            bv = x;
            bi = v;
          }
        }
      float ov = __shfl_xor(bv, 16);
      int oi = __shfl_xor(bi, 16);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      ov = __shfl_xor(bv, 32);
      oi = __shfl_xor(bi, 32);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      const int rel = bi - (v0 + 4 * g);
      if (bi != INT_MAX && rel >= 0 && (rel & 15) < 4 && (rel >> 4) < kLmMT)
        taken |= 1u << ((rel >> 4) * 4 + (rel & 3));
      if (g == 0 && t < T) {
        const size_t o = ((size_t)wglob * T + t) * p.k + r;
        p.part_val[o] = bv;
        p.part_idx[o] = bi;
      }
    }
  }
}

template <typename V, typename Op>
__device__ __forceinline__ V block_reduce256(V v, V* red, Op op) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return op(op(red[0], red[1]), op(red[2], red[3]));
}

__device__ __forceinline__ void block_best256(float& v, int& i, float* rv, int* ri) {
  wave_best(v, i);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    rv[threadIdx.x >> 6] = v;
    ri[threadIdx.x >> 6] = i;
  }
  __syncthreads();
  v = rv[0];
  i = ri[0];
  for (int w = 1; w < 4; ++w)
    if (better(rv[w], ri[w], v, i)) { v = rv[w]; i = ri[w]; }
}

// One workgroup per feature row: combine the per-wave statistics and top-k.
//
// Each wave's list is sorted by (logit desc, index asc).  Let theta be the
// k-th best of the lists' first entries: those k entries are all at least
// theta, so every member of the global top-k is too, and in each list only the
// prefix not worse than theta can contribute.  The selections run inside
// single waves (shuffle reductions, no workgroup barriers): each wave finds
// the top k of the first entries it holds, theta is the k-th best of those
// 4k candidates, survivors are gathered in LDS, and wave 0 picks the final k
// by repeated "best candidate strictly after the previous pick".  If more
// survive than LDS holds, wave 0 rescans every candidate instead (same result).
constexpr int kMergeCap = 4096;
constexpr int kMergePer = 12;     // lists per lane kept in registers (nw <= 3072)

__global__ __launch_bounds__(256) void lmhead_merge_kernel(
    const float2* __restrict__ part_stat, const float* __restrict__ part_val,
    const int32_t* __restrict__ part_idx, int nw, int T, int k, int32_t* __restrict__ topk_id,
    float* __restrict__ topk_logp, float* __restrict__ lse) {
  __shared__ float redf[4];
  __shared__ float cv[4 * EAGLE_MAX_TOPK];
  __shared__ int ci[4 * EAGLE_MAX_TOPK];
  __shared__ float sv[kMergeCap];
  __shared__ int si[kMergeCap];
  __shared__ int scount;
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float M = -INFINITY;
  for (int w = threadIdx.x; w < nw; w += 256) M = fmaxf(M, part_stat[(size_t)w * T + t].x);
  M = block_reduce256(M, redf, [](float a, float b) { return fmaxf(a, b); });
  float S = 0.f;
  for (int w = threadIdx.x; w < nw; w += 256) {
    const float2 st = part_stat[(size_t)w * T + t];
    if (st.y > 0.f) S += st.y * expf(st.x - M);
  }
  S = block_reduce256(S, redf, [](float a, float b) { return a + b; });
  const float L = M + logf(S);
  if (threadIdx.x == 0) scount = 0;

  // each wave: top k of the first entries of its lists (thread q-th list w =
  // threadIdx.x + 256 q)
  const bool inreg = nw <= 256 * kMergePer;
  float hv[kMergePer];
  int hi[kMergePer];
#pragma unroll
  for (int q = 0; q < kMergePer; ++q) {
    const int w = threadIdx.x + 256 * q;
    hv[q] = -INFINITY;
    hi[q] = INT_MAX;
    if (inreg && w < nw) {
      const size_t o = ((size_t)w * T + t) * k;
      hv[q] = part_val[o];
      hi[q] = part_idx[o];
    }
  }
  {
    float lastv = INFINITY;
    int lasti = -1;
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int bi = INT_MAX;
      if (inreg) {
#pragma unroll
        for (int q = 0; q < kMergePer; ++q)
          if (better(lastv, lasti, hv[q], hi[q]) && better(hv[q], hi[q], bv, bi)) {
            bv = hv[q];
            bi = hi[q];
          }
      } else {
        for (int w = threadIdx.x; w < nw; w += 256) {
          const size_t o = ((size_t)w * T + t) * k;
          const float v = part_val[o];
          const int i = part_idx[o];
          if (better(lastv, lasti, v, i) && better(v, i, bv, bi)) {
            bv = v;
            bi = i;
          }
        }
      }
      wave_best(bv, bi);
      if (lane == 0) {
        cv[wave * k + r] = bv;
        ci[wave * k + r] = bi;
      }
      lastv = bv;
      lasti = bi;
    }
  }
  __syncthreads();
  // theta = k-th best of the 4k wave candidates (every wave computes it)
  float thv = -INFINITY;
  int thi = INT_MAX;
  if (nw >= k) {
    const float myv = lane < 4 * k ? cv[lane] : -INFINITY;
    const int myi = lane < 4 * k ? ci[lane] : INT_MAX;
    const float myv2 = lane + 64 < 4 * k ? cv[lane + 64] : -INFINITY;
    const int myi2 = lane + 64 < 4 * k ? ci[lane + 64] : INT_MAX;
    const float myv3 = lane + 128 < 4 * k ? cv[lane + 128] : -INFINITY;
    const int myi3 = lane + 128 < 4 * k ? ci[lane + 128] : INT_MAX;
    const float myv4 = lane + 192 < 4 * k ? cv[lane + 192] : -INFINITY;
    const int myi4 = lane + 192 < 4 * k ? ci[lane + 192] : INT_MAX;
    float lastv = INFINITY;
    int lasti = -1;
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int bi = INT_MAX;
      if (better(lastv, lasti, myv, myi) && better(myv, myi, bv, bi)) { bv = myv; bi = myi; }
      if (better(lastv, lasti, myv2, myi2) && better(myv2, myi2, bv, bi)) { bv = myv2; bi = myi2; }
      if (better(lastv, lasti, myv3, myi3) && better(myv3, myi3, bv, bi)) { bv = myv3; bi = myi3; }
      if (better(lastv, lasti, myv4, myi4) && better(myv4, myi4, bv, bi)) { bv = myv4; bi = myi4; }
      wave_best(bv, bi);
      lastv = bv;
      lasti = bi;
    }
    thv = lastv;
    thi = lasti;
  }
  // survivors: the list prefixes not worse than theta (a list whose first
  // entry, already in registers, is worse than theta is skipped unread)
#pragma unroll
  for (int q = 0; q < kMergePer; ++q) {
    const int w = threadIdx.x + 256 * q;
    if (!inreg || w >= nw || better(thv, thi, hv[q], hi[q])) continue;
    const size_t o = ((size_t)w * T + t) * k;
    for (int j = 0; j < k; ++j) {
      const float v = j == 0 ? hv[q] : part_val[o + j];
      const int i = j == 0 ? hi[q] : part_idx[o + j];
      if (better(thv, thi, v, i)) break;      // worse than theta: the rest of the list too
      const int slot = atomicAdd(&scount, 1);
      if (slot < kMergeCap) {
        sv[slot] = v;
        si[slot] = i;
      }
    }
  }
  if (!inreg) {
    for (int w = threadIdx.x; w < nw; w += 256) {
      const size_t o = ((size_t)w * T + t) * k;
      for (int j = 0; j < k; ++j) {
        const float v = part_val[o + j];
        const int i = part_idx[o + j];
        if (better(thv, thi, v, i)) break;
        const int slot = atomicAdd(&scount, 1);
        if (slot < kMergeCap) {
          sv[slot] = v;
          si[slot] = i;
        }
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const int ns = scount;
  const bool fits = ns <= kMergeCap;
  float lastv = INFINITY;
  int lasti = -1;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (fits) {
      for (int c = lane; c < ns; c += 64) {
        const float v = sv[c];
        const int i = si[c];
        if (better(lastv, lasti, v, i) && better(v, i, bv, bi)) {
          bv = v;
          bi = i;
        }
      }
    } else {
      const int n = nw * k;
      for (int c = lane; c < n; c += 64) {
        const int w = c / k;
        const size_t o = ((size_t)w * T + t) * k + (c - w * k);
        const float v = part_val[o];
        const int i = part_idx[o];
        if (better(lastv, lasti, v, i) && better(v, i, bv, bi)) {
          bv = v;
          bi = i;
        }
      }
    }
    wave_best(bv, bi);
    if (lane == 0) {
      topk_id[(size_t)t * k + r] = bi;
      topk_logp[(size_t)t * k + r] = bv - L;
    }
    lastv = bv;
    lasti = bi;
  }
  if (lane == 0) lse[t] = L;
}

// ---------------------------------------------------------------- fp32 path

__global__ __launch_bounds__(256) void lmhead_f32_logits_kernel(
    const float* __restrict__ f, const float* __restrict__ W, int T, int d, int V,
    float* __restrict__ logits) {
  __shared__ float fsm[1024];
  const int t = blockIdx.y;
  const int v = blockIdx.x * 256 + threadIdx.x;
  float acc = 0.f;
  for (int k0 = 0; k0 < d; k0 += 1024) {
    const int n = min(1024, d - k0);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) fsm[i] = f[(size_t)t * d + k0 + i];
    __syncthreads();
    if (v < V) {
      const float* w = W + (size_t)v * d + k0;
      for (int i = 0; i < n; ++i) acc = fmaf(fsm[i], w[i], acc);
    }
  }
  if (v < V) logits[(size_t)t * V + v] = acc;
}

__global__ __launch_bounds__(256) void rows_topk_kernel(
    const float* __restrict__ logits, int V, int k, int32_t* __restrict__ topk_id,
    float* __restrict__ topk_logp, float* __restrict__ lse) {
  __shared__ float redf[4];
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int t = blockIdx.x;
  const float* row = logits + (size_t)t * V;
  float M = -INFINITY;
  for (int v = threadIdx.x; v < V; v += 256) M = fmaxf(M, row[v]);
  M = block_reduce256(M, redf, [](float a, float b) { return fmaxf(a, b); });
  float S = 0.f;
  for (int v = threadIdx.x; v < V; v += 256) S += expf(row[v] - M);
  S = block_reduce256(S, redf, [](float a, float b) { return a + b; });
  const float L = M + logf(S);
  float lastv = INFINITY;
  int lasti = -1;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int v = threadIdx.x; v < V; v += 256) {
      const float x = row[v];
      if (better(lastv, lasti, x, v) && better(x, v, bv, bi)) {
        bv = x;
        bi = v;
      }
    }
    block_best256(bv, bi, rv, ri);
    if (threadIdx.x == 0) {
      topk_id[(size_t)t * k + r] = bi;
      topk_logp[(size_t)t * k + r] = bv - L;
    }
    lastv = bv;
    lasti = bi;
  }
  if (threadIdx.x == 0) lse[t] = L;
}

// ---------------------------------------------------------------- host side

struct LmLayout {
  size_t stat_off, val_off, idx_off, logits_off, total;
  int nw;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static LmLayout lm_layout(int T, int V, int k, eagle_dtype dt) {
  LmLayout l{};
  if (dt == EAGLE_BF16) {
    const int rows_block = 16 * lm_mt(T) * kLmWaves;
    l.nw = ((V + rows_block - 1) / rows_block) * kLmWaves;
    l.stat_off = 0;
    l.val_off = align256((size_t)l.nw * T * sizeof(float2));
    l.idx_off = l.val_off + align256((size_t)l.nw * T * k * sizeof(float));
    l.total = l.idx_off + align256((size_t)l.nw * T * k * sizeof(int32_t));
  } else {
    l.logits_off = 0;
    l.total = align256((size_t)T * V * sizeof(float));
  }
  return l;
}

template <int NT, int MT>
static void launch_lm(const LmParams& p, hipStream_t s) {
  const int rows_block = 16 * MT * kLmWaves;
  hipLaunchKernelGGL((lmhead_bf16_kernel<NT, MT>), dim3((p.V + rows_block - 1) / rows_block),
                     dim3(256), 0, s, p);
}

}  // namespace eagle

extern "C" size_t eagle_lmhead_topk_workspace(int32_t T, int32_t d, int32_t V, int32_t k,
                                              eagle_dtype dt) {
  (void)d;
  if (T < 1 || V < 1 || k < 1) return 0;
  return eagle::lm_layout(T, V, k, dt).total;
}

extern "C" int eagle_lmhead_topk(const void* f, const void* W, int32_t T, int32_t d, int32_t V,
                                 int32_t k, eagle_dtype dt, int32_t* topk_id, float* topk_logp,
                                 float* lse, float* logits, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
  using namespace eagle;
  EAGLE_REQUIRE(f && W && topk_id && topk_logp && lse && workspace, EAGLE_EINVAL);
  EAGLE_REQUIRE(T >= 1 && T <= EAGLE_MAX_TREE && d >= 1 && V >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(k >= 1 && k <= EAGLE_MAX_TOPK && k <= V, EAGLE_EINVAL);
  EAGLE_REQUIRE(((uintptr_t)workspace & 255) == 0, EAGLE_EINVAL);
  const LmLayout l = lm_layout(T, V, k, dt);
  EAGLE_REQUIRE(ws_bytes >= l.total, EAGLE_EWORKSPACE);
  char* ws = (char*)workspace;
  if (dt == EAGLE_BF16) {
    EAGLE_REQUIRE(d % kWsKG == 0, EAGLE_EUNSUPPORTED);
    EAGLE_REQUIRE(((uintptr_t)f & 15) == 0 && ((uintptr_t)W & 15) == 0, EAGLE_EINVAL);
    EAGLE_REQUIRE(!logits || ((uintptr_t)logits & 15) == 0, EAGLE_EINVAL);
    LmParams p{(const bf16_t*)f, (const bf16_t*)W, T, d, V, k, logits,
               (float2*)(ws + l.stat_off), (float*)(ws + l.val_off), (int32_t*)(ws + l.idx_off)};
    const int nt = (T + 15) / 16;
    static_assert(lm_mt(16) == 8 && lm_mt(64) == 2 && lm_mt(128) == 2 && lm_mt(129) == 1,
                  "tile choice");
    if (nt <= 1) launch_lm<1, 8>(p, stream);
    else if (nt <= 2) launch_lm<2, 2>(p, stream);
    else if (nt <= 4) launch_lm<4, 2>(p, stream);
    else if (nt <= 8) launch_lm<8, 2>(p, stream);
    else launch_lm<16, 1>(p, stream);
    EAGLE_LAUNCH_CHECK();
    hipLaunchKernelGGL(lmhead_merge_kernel, dim3(T), dim3(256), 0, stream, p.part_stat,
                       p.part_val, p.part_idx, l.nw, T, k, topk_id, topk_logp, lse);
  } else if (dt == EAGLE_F32) {
    float* lg = logits ? logits : (float*)(ws + l.logits_off);
    hipLaunchKernelGGL(lmhead_f32_logits_kernel, dim3((V + 255) / 256, T), dim3(256), 0, stream,
                       (const float*)f, (const float*)W, T, d, V, lg);
    EAGLE_LAUNCH_CHECK();
    hipLaunchKernelGGL(rows_topk_kernel, dim3(T), dim3(256), 0, stream, lg, V, k, topk_id,
                       topk_logp, lse);
  } else {
    return EAGLE_EINVAL;
  }
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
