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
//     feature rows as N (16 per tile, NT tiles), from the shared weight-streaming
//     core (wstream.h).  With 8 tiles per wave W is read in runs of 256 bytes
//     per row with non-temporal loads and passed through a wave-private LDS tile
//     into the operand layout (6.0 against 5.5 TB/s at T = 10 for W read
//     straight into operands, 16 rows x 64 bytes per load instruction); with 4
//     tiles the LDS it would need leaves one workgroup per CU, so W goes
//     straight into A operands.
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
#include <mutex>

#include "wstream.h"

namespace eagle {

constexpr int kLmWaves = 4;
// Largest k whose four per-wave lists fit the X staging buffer for the
// workgroup-level merge: 4 waves x 16 NT rows x (k + 1) x 8 bytes against
// 2 x 16 NT x 136 x 2 bytes.
constexpr int kLmBlockK = 16;
static_assert(2 * 16 * kWsLds * 2 >= 4 * 16 * (kLmBlockK + 1) * 8, "lists exceed staging LDS");
static_assert(sizeof(selkey_t) == 8, "key size");

// W tiles of 16 rows per wave: 8 (128 rows, one 4-wave workgroup per CU) up to
// T = 64, which keeps the most weight bytes in flight per wave; fewer as more
// feature rows need accumulator registers.  Eight tiles at 32 < T <= 64 fit
// because W then passes through registers one k step at a time (row runs,
// wstream_mfma_rr) and the accumulators may live in AGPRs (this file is built
// with the MFMA results in VGPR form, spilling to AGPRs: none to memory).
// Measured at V = 128256, d = 4096: T = 32 takes 197 us with eight tiles
// straight into operands and 243 us with four; T = 64 with logits 268 us with
// four tiles and 213 us with eight in row runs.
__host__ __device__ constexpr int lm_mt(int T) {
  return T <= 64 ? 8 : (T <= 128 ? 2 : 1);
}

// The feature-row tiles a launch is compiled for (1, 2, 4, 8 or 16 of 16 rows).
// The launch and the workspace layout both take the tile count from here and
// the W tiles from lm_mt(16 * lm_nt(T)), so the two can never disagree.
__host__ __device__ constexpr int lm_nt(int T) {
  return T <= 16 ? 1 : (T <= 32 ? 2 : (T <= 64 ? 4 : (T <= 128 ? 8 : 16)));
}

struct LmParams {
  const bf16_t* f;
  const bf16_t* W;
  int T, d, V, k;
  float* logits;
  float2* part_stat;   // [T][nb] (max, sum exp(l - max))
  selkey_t* part_key;  // [T][nb][k] sorted selection keys
  RowNorm in;          // deferred RMSNorm of the feature rows (in.ssq null: none)
  selkey_t* thr;       // [T] per row, a key that is at most its k-th largest
                       // (0 between calls; see the epilogue)
};

template <int NT, int kLmMT>
__global__ __launch_bounds__(256, (kLmMT >= 8 || NT >= 16 ? 1 : 2)) void lmhead_bf16_kernel(
    LmParams p) {
  constexpr int kLmRowsWave = 16 * kLmMT;
  constexpr int kLmRowsBlock = kLmRowsWave * kLmWaves;
  // (8 W tiles with 4 or more feature tiles: one activation buffer, so that
  // the W tiles of the row-run path fit)
  // Row-run weight streaming (through a wave-private LDS tile) for eight
  // tiles per wave, and for four at T <= 16 (the tile count that lm_mt_for
  // picks for vocabularies past one round of 512-row workgroups).
  constexpr bool kRowRuns = kLmMT == 8 || (kLmMT == 4 && NT == 1);
  constexpr bool kXSingle = kLmMT == 8 && NT >= 4;
  __shared__ __attribute__((aligned(16))) bf16_t fs[kXSingle ? ws_lds_elems<NT>() / 2
                                                             : ws_lds_elems<NT>()];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index as a scalar, so that the row-run path's per-tile buffer
  // descriptors are uniform (held in SGPRs, no per-load waterfall loop)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int v0 = blockIdx.x * kLmRowsBlock + wave * kLmRowsWave;

  const bf16_t* wrow[kLmMT];
#pragma unroll
  for (int mt = 0; mt < kLmMT; ++mt) {
    const int v = min(v0 + mt * 16 + r16, p.V - 1);
    wrow[mt] = p.W + (size_t)v * p.d + g * 8;
  }
  // deferred RMSNorm of the feature rows: the first partial sums are loaded
  // before the main loop and the sums finished after it.  2^tsh consecutive
  // lanes share a row (16 at T <= 16, 8 at T <= 32, ..., 1 at T > 128): lane
  // q0 of row rm takes partials q0, q0 + 2^tsh, ...
  __shared__ float rsc[EAGLE_MAX_TREE];
  const int tsh = p.T <= 16 ? 4 : p.T <= 32 ? 3 : p.T <= 64 ? 2 : p.T <= 128 ? 1 : 0;
  const int rm = tid >> tsh;
  const int q0 = tid & ((1 << tsh) - 1);
  const bool has_in = p.in.ssq && rm < p.T;
  float in_part[kPartBatch];
  if (has_in) strided_load(p.in.ssq + rm, p.in.parts, (size_t)p.T, q0, 1 << tsh, in_part);
  // (4 x 4 tiles: no registers to spare for the partials across the loop)
  constexpr bool kInAcross = !(NT == 4 && kLmMT == 4);
  float in_ss = 0.f;
  if (!kInAcross && has_in)
    in_ss = strided_finish(p.in.ssq + rm, p.in.parts, (size_t)p.T, q0, 1 << tsh, in_part);

  f32x4 acc[kLmMT][NT];
  // W tiles of the row-run path; after the main loop, the epilogue's lists
  __shared__ __attribute__((aligned(16))) char wlds[kRowRuns ? kLmWaves : 1][kLmMT * 4096];
  if constexpr (kRowRuns) {
    // row-run loads through a wave-private LDS tile
    int trow[kLmMT], wsel[kLmMT];
#pragma unroll
    for (int mt = 0; mt < kLmMT; ++mt) {
      trow[mt] = v0 + mt * 16;
      wsel[mt] = 0;
    }
    wstream_mfma_rr<NT, kLmMT, kXSingle>(p.W, nullptr, p.V, p.d, trow, wsel, p.f, p.d, p.T, p.d,
                                         fs, wlds[wave], acc);
  } else {
    wstream_mfma<NT, kLmMT>(wrow, p.f, p.d, p.T, p.d, fs, acc);
  }

  if (p.in.ssq) {
    if (kInAcross && has_in)
      in_ss = strided_finish(p.in.ssq + rm, p.in.parts, (size_t)p.T, q0, 1 << tsh, in_part);
    // sum over the row's lanes (pairs, quads, 8, 16: a butterfly inside each group)
    if (tsh > 0) in_ss += dpp_move<kDppQuadXor1>(in_ss);
    if (tsh > 1) in_ss += dpp_move<kDppQuadXor2>(in_ss);
    if (tsh > 2) in_ss += dpp_move<kDppHalfMirror>(in_ss);
    if (tsh > 3) in_ss += dpp_move<kDppRowMirror>(in_ss);
    if (rm < p.T && q0 == 0) rsc[rm] = 1.0f / sqrtf(in_ss / (float)p.in.n + p.in.eps);
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int t = nt * 16 + r16;
      const float r = t < p.T ? rsc[t] : 1.0f;
#pragma unroll
      for (int mt = 0; mt < kLmMT; ++mt) acc[mt][nt] = acc[mt][nt] * r;
    }
  }

  // ---- epilogue.  Lane (g, r16) holds, for tile (mt, nt), the logits of
  // vocabulary rows v0 + 16 mt + 4 g + j (j < 4) for feature row 16 nt + r16.
  const int T = p.T;
  const int V = p.V;
  const int wglob = blockIdx.x * kLmWaves + wave;
  if (p.logits) {
    // With at most 2 tiles per wave the workgroup's [16 NT][rows] fp32 tile
    // fits the staging buffer: it goes through LDS so that every store writes
    // whole 16-byte pieces of contiguous row segments (RB floats per row);
    // otherwise lanes store their 4-logit pieces directly.
    constexpr int RB = kLmRowsBlock;
    constexpr int RBP = RB + 4;     // padded LDS row
    constexpr bool kStage = 16 * NT * RBP * 4 <= ws_lds_elems<NT>() * 2;
    if (kStage) {
      float* lt = (float*)fs;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < kLmMT; ++mt)
          *(f32x4*)(lt + (nt * 16 + r16) * RBP + wave * kLmRowsWave + mt * 16 + 4 * g) =
              acc[mt][nt];
      __syncthreads();
      const int vblk = blockIdx.x * RB;
      const bool vec = (V & 3) == 0;
      for (int e = tid; e < 16 * NT * (RB / 4); e += 256) {
        const int t = e / (RB / 4);
        const int c = e - t * (RB / 4);
        const int v = vblk + 4 * c;
        if (t >= T || v >= V) continue;
        const f32x4 x = *(const f32x4*)(lt + t * RBP + 4 * c);
        float* out = p.logits + (size_t)t * V + v;
        if (vec && v + 3 < V) {
          *(f32x4*)out = x;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (v + j < V) out[j] = x[j];
        }
      }
      __syncthreads();   // the staging buffer is reused below
    } else {
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
  }
  // Per wave and feature row: (max, sum exp(l - max)) and the top-k as
  // selection keys, by k rounds of "largest key below the previous pick".
  // With k <= kLmBlockK the four waves' sorted lists go to LDS (the W tiles on
  // the row-run path, else the X staging buffer: both free after the main
  // loop) and are merged into one list per workgroup; otherwise every wave
  // writes its own.
  const bool block_lists = p.k <= kLmBlockK;
  constexpr int TP = 16 * NT;
  static_assert(!kRowRuns || kLmWaves * kLmMT * 4096 >= 4 * TP * (kLmBlockK + 1) * 8,
                "lists exceed the W tiles' LDS");
  selkey_t* lk = kRowRuns ? (selkey_t*)&wlds[0][0] : (selkey_t*)fs;   // [4][TP][k]
  float2* ls = (float2*)(lk + 4 * TP * p.k);    // [4][TP]
  const int nb = block_lists ? gridDim.x : gridDim.x * kLmWaves;
  const int list = block_lists ? blockIdx.x : wglob;
  // A key below row t's k-th largest over the whole vocabulary is never
  // needed.  p.thr[t] is a lower bound of that k-th largest: the largest k-th
  // entry of any list finished so far in this call (every list is a set of
  // keys of row t, so its k-th entry has k keys at or above it).  A list
  // therefore keeps only keys >= the bound it reads, and its selection rounds
  // stop once every row of the wave has run out of them: the lists finished
  // last, which end the call, usually need a round or two instead of k.  The
  // merged top-k does not depend on the bounds read (every key of the row's
  // top-k is >= every bound), so the results stay identical from call to call.
  selkey_t thr[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = nt * 16 + r16;
    thr[nt] = t < T && p.k > 0 ? __hip_atomic_load(p.thr + t, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : ~0ull;
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
    m = rows_max(m);
    // exp(l - m) as the hardware base-2 exponential of (l - m) log2(e)
    // (about 1e-6 relative: far below the bf16 rounding of the logits)
    float s = 0.f;
#pragma unroll
    for (int mt = 0; mt < kLmMT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v0 + mt * 16 + 4 * g + j < V)
          s += __builtin_amdgcn_exp2f((acc[mt][nt][j] - m) * 1.4426950408889634f);
    s = rows_sum(s);
    if (g == 0) {
      if (block_lists) ls[wave * TP + t] = make_float2(m, s);
      else if (t < T) p.part_stat[(size_t)t * nb + list] = make_float2(m, s);
    }

    selkey_t last = ~0ull;
    for (int r = 0; r < p.k; ++r) {
      selkey_t best = 0;
#pragma unroll
      for (int mt = 0; mt < kLmMT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = v0 + mt * 16 + 4 * g + j;
          const selkey_t key = v < V ? sel_key(acc[mt][nt][j], v) : 0ull;
          best = ((key < last) & (key > best)) ? key : best;
        }
      best = rows_max_key(best);
      best = best >= thr[nt] ? best : 0ull;
      const bool more = __any(best != 0ull);
      // this round's entry, and none for the rounds skipped below
      for (int e = r; e < (more ? r + 1 : p.k); ++e) {
        const selkey_t x = e == r ? best : 0ull;
        if (g == 0) {
          if (block_lists) lk[(wave * TP + t) * p.k + e] = x;
          else if (t < T) p.part_key[((size_t)t * nb + list) * p.k + e] = x;
        }
      }
      if (!block_lists && r == p.k - 1 && g == 0 && t < T && best != 0ull)
        __hip_atomic_fetch_max(p.thr + t, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!more) break;
      last = best;
    }
  }
  if (!block_lists) return;
  __syncthreads();
  // Workgroup merge: lane (g, r16) of the wave that owns tile nt follows wave
  // g's sorted list of row 16 nt + r16; each round the largest of the four
  // heads (lanes r16, r16 + 16, r16 + 32, r16 + 48) wins and its owner
  // advances (keys of distinct vocabulary rows never tie).
  for (int nt = wave; nt < NT; nt += kLmWaves) {
    const int t = nt * 16 + r16;
    const float2 st = ls[g * TP + t];
    const float M = rows_max(st.x);
    const float S = rows_sum(st.y > 0.f ? st.y * expf(st.x - M) : 0.f);
    if (g == 0 && t < T) p.part_stat[(size_t)t * nb + list] = make_float2(M, S);
    const selkey_t* my = lk + (g * TP + t) * p.k;
    int ptr = 0;
    selkey_t h = my[0];
    for (int r = 0; r < p.k; ++r) {
      const selkey_t b = rows_max_key(h);
      const bool adv = (h == b) & (b != 0ull);
      ptr += adv ? 1 : 0;
      const selkey_t nxt = my[min(ptr, p.k - 1)];
      h = adv ? (ptr < p.k ? nxt : 0ull) : h;
      const bool more = __any(b != 0ull);
      for (int e = r; e < (more ? r + 1 : p.k); ++e)
        if (g == 0 && t < T) p.part_key[((size_t)t * nb + list) * p.k + e] = e == r ? b : 0ull;
      if (r == p.k - 1 && g == 0 && t < T && b != 0ull)   // the list's k-th entry
        __hip_atomic_fetch_max(p.thr + t, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!more) break;
    }
  }
}

template <typename V, typename Op>
__device__ __forceinline__ V block_reduce256(V v, V* red, Op op) {
  v = wave_reduce(v, op);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return op(op(red[0], red[1]), op(red[2], red[3]));
}

// One workgroup per feature row: combine the nb partial statistics and top-k
// lists of the row (stored contiguously: stat[t][nb], key[t][nb][k], each
// list sorted by descending selection key).
//
// lse: the (max, sum) pairs are folded with the usual rescaling, in a fixed
// assignment and reduction order.  Top-k: let theta be the k-th largest of
// the lists' first keys.  Those k keys are all at least theta, so every member
// of the row's top k is too, and only lists whose first key is not below
// theta can contribute: at most k of them (keys never tie).  theta comes from
// per-wave selections over first keys held in registers; the surviving lists
// are copied into LDS and wave 0 merges them, one list per lane, in k rounds.
// Rows with few short lists take a one-pass path (below).
constexpr int kMergeHeads = 16;   // first keys per thread held in registers

// (m, s) <- the pair for the union of both sets; a pair with s = 0 is empty.
// Select-based (no branches) and commutative: both orders give the same bits.
__device__ __forceinline__ void fold_stat(float& m, float& s, float m2, float s2) {
  const bool h1 = s > 0.f, h2 = s2 > 0.f;
  const float M = h1 ? (h2 ? fmaxf(m, m2) : m) : m2;
  const float a = h1 ? s * expf(m - M) : 0.f;
  const float b = h2 ? s2 * expf(m2 - M) : 0.f;
  m = (h1 | h2) ? M : m;
  s = a + b;
}

template <int CTRL>
__device__ __forceinline__ void fold_step(float& m, float& s) {
  const float m2 = dpp_move<CTRL>(m), s2 = dpp_move<CTRL>(s);
  fold_stat(m, s, m2, s2);
}

// fold_stat is commutative, so the butterfly leaves every lane the same pair.
__device__ __forceinline__ void fold_stat_wave(float& m, float& s) {
  fold_step<kDppQuadXor1>(m, s);
  fold_step<kDppQuadXor2>(m, s);
  fold_step<kDppHalfMirror>(m, s);
  fold_step<kDppRowMirror>(m, s);
  float ma, mb, sa, sb;
  swap16(m, ma, mb);
  swap16(s, sa, sb);
  fold_stat(ma, sa, mb, sb);
  swap32(ma, m, mb);
  swap32(sa, s, sb);
  fold_stat(m, s, mb, sb);
}

__global__ __launch_bounds__(256) void lmhead_merge_kernel(
    const float2* __restrict__ part_stat, const selkey_t* __restrict__ part_key, int nb, int T,
    int k, int32_t* __restrict__ topk_id, float* __restrict__ topk_logp,
    float* __restrict__ lse, selkey_t* __restrict__ thr) {
  __shared__ float2 red[4];
  __shared__ selkey_t ck[4 * EAGLE_MAX_TOPK];
  __shared__ int slist[EAGLE_MAX_TOPK];
  __shared__ int nsl;
  __shared__ selkey_t sk[EAGLE_MAX_TOPK * EAGLE_MAX_TOPK];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float2* st = part_stat + (size_t)t * nb;
  const selkey_t* pk = part_key + (size_t)t * nb * k;
  if (tid == 0) nsl = 0;
  // the main kernel is done with row t's bound: zero for the next call
  if (tid == 0) __hip_atomic_store(thr + t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // Short lists (nb <= 256, nb k <= 4096 keys): all keys go to LDS in one
  // pass and wave 0 merges every list directly, lane l following lists l,
  // l + 64, l + 128 and l + 192, with each list's next key read ahead.
  if (nb <= 256 && nb * k <= EAGLE_MAX_TOPK * EAGLE_MAX_TOPK) {
    {
      // every key load of the thread in flight before the first LDS store
      constexpr int KPT = EAGLE_MAX_TOPK * EAGLE_MAX_TOPK / 256;
      selkey_t kv[KPT];
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int c = tid + 256 * i;
        kv[i] = c < nb * k ? pk[c] : 0ull;
      }
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int c = tid + 256 * i;
        if (c < nb * k) sk[c] = kv[i];
      }
    }
    float m = -INFINITY, s = 0.f;
    for (int w = tid; w < nb; w += 256) {
      const float2 x = st[w];
      fold_stat(m, s, x.x, x.y);
    }
    fold_stat_wave(m, s);
    if (lane == 0) red[wave] = make_float2(m, s);
    __syncthreads();
    if (wave != 0) return;
    float M = red[0].x, S = red[0].y;
    for (int w = 1; w < 4; ++w) fold_stat(M, S, red[w].x, red[w].y);
    const float L = M + logf(S);
    selkey_t hq[4], nx[4];
    int ptr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int w = lane + 64 * q;
      ptr[q] = 0;
      hq[q] = w < nb && k > 0 ? sk[w * k] : 0ull;
      nx[q] = w < nb && k > 1 ? sk[w * k + 1] : 0ull;
    }
    for (int r = 0; r < k; ++r) {
      selkey_t h = hq[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) h = hq[q] > h ? hq[q] : h;
      const selkey_t b = wave_max_key(h);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int w = lane + 64 * q;
        const bool adv = (hq[q] == b) & (b != 0ull);
        ptr[q] += adv ? 1 : 0;
        hq[q] = adv ? nx[q] : hq[q];
        const int nxt = ptr[q] + 1;
        const selkey_t ahead = (w < nb && nxt < k) ? sk[w * k + nxt] : 0ull;
        nx[q] = adv ? ahead : nx[q];
      }
      if (lane == 0) {
        topk_id[(size_t)t * k + r] = b ? key_index(b) : -1;
        topk_logp[(size_t)t * k + r] = b ? key_value(b) - L : -INFINITY;
      }
    }
    if (lane == 0) lse[t] = L;
    return;
  }

  // first keys (issued before the statistics pass so the loads overlap)
  const bool inreg = nb <= 256 * kMergeHeads;
  selkey_t hk[kMergeHeads];
#pragma unroll
  for (int q = 0; q < kMergeHeads; ++q) {
    const int w = tid + 256 * q;
    hk[q] = (inreg && w < nb) ? pk[(size_t)w * k] : 0ull;
  }

  float m = -INFINITY, s = 0.f;
  for (int w = tid; w < nb; w += 256) {
    const float2 x = st[w];
    fold_stat(m, s, x.x, x.y);
  }
  fold_stat_wave(m, s);
  if (lane == 0) red[wave] = make_float2(m, s);

  // per wave: the k largest first keys it holds
  {
    selkey_t last = ~0ull;
    for (int r = 0; r < k; ++r) {
      selkey_t b = 0;
      if (inreg) {
#pragma unroll
        for (int q = 0; q < kMergeHeads; ++q) b = ((hk[q] < last) & (hk[q] > b)) ? hk[q] : b;
      } else {
        for (int w = tid; w < nb; w += 256) {
          const selkey_t x = pk[(size_t)w * k];
          b = ((x < last) & (x > b)) ? x : b;
        }
      }
      b = wave_max_key(b);
      if (lane == 0) ck[wave * k + r] = b;
      last = b;
    }
  }
  __syncthreads();
  float M = red[0].x, S = red[0].y;
  for (int w = 1; w < 4; ++w) fold_stat(M, S, red[w].x, red[w].y);
  const float L = M + logf(S);

  // theta = k-th largest of the 4k wave candidates (0 if fewer exist)
  selkey_t theta = ~0ull;
  {
    selkey_t c4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      c4[c] = e < 4 * k ? ck[e] : 0ull;
    }
    for (int r = 0; r < k; ++r) {
      selkey_t b = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) b = ((c4[c] < theta) & (c4[c] > b)) ? c4[c] : b;
      theta = wave_max_key(b);
    }
  }
  // lists whose first key is real and not below theta
  if (inreg) {
#pragma unroll
    for (int q = 0; q < kMergeHeads; ++q)
      if (hk[q] != 0ull && hk[q] >= theta) {
        const int slot = atomicAdd(&nsl, 1);
        if (slot < EAGLE_MAX_TOPK) slist[slot] = tid + 256 * q;
      }
  } else {
    for (int w = tid; w < nb; w += 256) {
      const selkey_t x = pk[(size_t)w * k];
      if (x != 0ull && x >= theta) {
        const int slot = atomicAdd(&nsl, 1);
        if (slot < EAGLE_MAX_TOPK) slist[slot] = w;
      }
    }
  }
  __syncthreads();
  const int ns = min(nsl, EAGLE_MAX_TOPK);
  for (int c = tid; c < ns * k; c += 256) {
    const int j = c / k;
    sk[c] = pk[(size_t)slist[j] * k + (c - j * k)];
  }
  __syncthreads();
  if (wave != 0) return;
  // k-way merge: lane j follows surviving list j
  int ptr = 0;
  selkey_t h = lane < ns ? sk[lane * k] : 0ull;
  for (int r = 0; r < k; ++r) {
    const selkey_t b = wave_max_key(h);
    const bool adv = (h == b) & (b != 0ull);
    ptr += adv ? 1 : 0;
    const selkey_t nxt = lane < ns ? sk[lane * k + min(ptr, k - 1)] : 0ull;
    h = adv ? (ptr < k ? nxt : 0ull) : h;
    if (lane == 0) {
      topk_id[(size_t)t * k + r] = b ? key_index(b) : -1;
      topk_logp[(size_t)t * k + r] = b ? key_value(b) - L : -INFINITY;
    }
  }
  if (lane == 0) lse[t] = L;
}

// ---------------------------------------------------------------- fp32 path

__global__ __launch_bounds__(256) void lmhead_f32_logits_kernel(
    const float* __restrict__ f, const float* __restrict__ W, int T, int d, int V, RowNorm in,
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
  if (in.ssq) acc *= row_norm_scale(in, T, t);
  if (v < V) logits[(size_t)t * V + v] = acc;
}

__global__ __launch_bounds__(256) void rows_topk_kernel(
    const float* __restrict__ logits, int V, int k, int32_t* __restrict__ topk_id,
    float* __restrict__ topk_logp, float* __restrict__ lse) {
  __shared__ float redf[4];
  const int t = blockIdx.x;
  const float* row = logits + (size_t)t * V;
  float M = -INFINITY;
  for (int v = threadIdx.x; v < V; v += 256) M = fmaxf(M, row[v]);
  M = block_reduce256(M, redf, [](float a, float b) { return fmaxf(a, b); });
  float S = 0.f;
  for (int v = threadIdx.x; v < V; v += 256) S += expf(row[v] - M);
  S = block_reduce256(S, redf, [](float a, float b) { return a + b; });
  const float L = M + logf(S);
  __shared__ selkey_t redk[4];
  selkey_t last = ~0ull;
  for (int r = 0; r < k; ++r) {
    selkey_t b = 0;
    for (int v = threadIdx.x; v < V; v += 256) {
      const selkey_t x = sel_key(row[v], v);
      b = ((x < last) & (x > b)) ? x : b;
    }
    b = block_reduce256(b, redk, [](selkey_t x, selkey_t y) { return kmax(x, y); });
    if (threadIdx.x == 0) {
      topk_id[(size_t)t * k + r] = b ? key_index(b) : -1;
      topk_logp[(size_t)t * k + r] = b ? key_value(b) - L : -INFINITY;
    }
    last = b;
  }
  if (threadIdx.x == 0) lse[t] = L;
}

// ---------------------------------------------------------------- host side

struct LmLayout {
  size_t thr_off, stat_off, key_off, logits_off, total;
  int nb;   // partial lists per feature row
};

// bf16 path: the per-row key bounds sit first, at a fixed place for every T
constexpr size_t kLmThrBytes = EAGLE_MAX_TREE * sizeof(selkey_t);

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kLmCUs = 256;   // MI355X compute units

// W tiles per wave for a launch: lm_mt, except that eight tiles (512 rows per
// workgroup, one workgroup per CU) are traded for four (two per CU) when the
// vocabulary needs more than one round of kLmCUs workgroups: at V = 152064
// eight tiles leave 41 workgroups for a second round (T = 10: 246 us with
// four tiles in the operand layout, 214 us with four on row runs).  The launch and the
// workspace layout both take the tile count from here.
static int lm_mt_for(int T, int V) {
  const int mt = lm_mt(16 * lm_nt(T));
  return mt == 8 && (V + 511) / 512 > kLmCUs ? 4 : mt;
}

static LmLayout lm_layout(int T, int V, int k, eagle_dtype dt) {
  LmLayout l{};
  if (dt == EAGLE_BF16) {
    const int rows_block = 16 * lm_mt_for(T, V) * kLmWaves;
    l.nb = ((V + rows_block - 1) / rows_block) * (k <= kLmBlockK ? 1 : kLmWaves);
    l.thr_off = 0;
    l.stat_off = kLmThrBytes;
    l.key_off = l.stat_off + align256((size_t)l.nb * T * sizeof(float2));
    l.total = l.key_off + align256((size_t)l.nb * T * k * sizeof(selkey_t));
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
  if (T < 1 || V < 1 || k < 0) return 0;
  return eagle::lm_layout(T, V, k, dt).total;
}

namespace eagle {

// The body of both entry points: arguments checked, then the launches, with
// `ws` holding the partial lists (bf16) or the fp32 logits when the caller
// passes none.
static int lm_run(const void* f, const void* W, int32_t T, int32_t d, int32_t V, int32_t k,
                  eagle_dtype dt, const float* in_ssq, int32_t in_parts, float in_eps,
                  int32_t* topk_id, float* topk_logp, float* lse, float* logits, char* ws,
                  size_t ws_bytes, hipStream_t stream) {
  EAGLE_REQUIRE(f && W && lse && ws && (k == 0 || (topk_id && topk_logp)), EAGLE_EINVAL);
  EAGLE_REQUIRE(!in_ssq || (in_parts >= 1 && in_eps >= 0.0f), EAGLE_EINVAL);
  const RowNorm rn{in_ssq, in_ssq ? in_parts : 0, d, in_eps};
  EAGLE_REQUIRE(T >= 1 && T <= EAGLE_MAX_TREE && d >= 1 && V >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(k >= 0 && k <= EAGLE_MAX_TOPK && k <= V, EAGLE_EINVAL);
  EAGLE_REQUIRE(((uintptr_t)ws & 255) == 0, EAGLE_EINVAL);
  const LmLayout l = lm_layout(T, V, k, dt);
  EAGLE_REQUIRE(ws_bytes >= l.total, EAGLE_EWORKSPACE);
  if (dt == EAGLE_BF16) {
    EAGLE_REQUIRE(d % kWsKG == 0, EAGLE_EUNSUPPORTED);
    EAGLE_REQUIRE(((uintptr_t)f & 15) == 0 && ((uintptr_t)W & 15) == 0, EAGLE_EINVAL);
    EAGLE_REQUIRE(!logits || ((uintptr_t)logits & 15) == 0, EAGLE_EINVAL);
    LmParams p{(const bf16_t*)f, (const bf16_t*)W, T, d, V, k, logits,
               (float2*)(ws + l.stat_off), (selkey_t*)(ws + l.key_off), rn,
               (selkey_t*)(ws + l.thr_off)};
    const bool eight = lm_mt_for(T, V) == 8;
    switch (lm_nt(T)) {
      case 1: eight ? launch_lm<1, 8>(p, stream) : launch_lm<1, 4>(p, stream); break;
      case 2: eight ? launch_lm<2, 8>(p, stream) : launch_lm<2, 4>(p, stream); break;
      case 4: eight ? launch_lm<4, 8>(p, stream) : launch_lm<4, 4>(p, stream); break;
      case 8: launch_lm<8, lm_mt(128)>(p, stream); break;
      default: launch_lm<16, lm_mt(256)>(p, stream); break;
    }
    EAGLE_LAUNCH_CHECK();
    hipLaunchKernelGGL(lmhead_merge_kernel, dim3(T), dim3(256), 0, stream, p.part_stat,
                       p.part_key, l.nb, T, k, topk_id, topk_logp, lse, p.thr);
  } else if (dt == EAGLE_F32) {
    float* lg = logits ? logits : (float*)(ws + l.logits_off);
    hipLaunchKernelGGL(lmhead_f32_logits_kernel, dim3((V + 255) / 256, T), dim3(256), 0, stream,
                       (const float*)f, (const float*)W, T, d, V, rn, lg);
    EAGLE_LAUNCH_CHECK();
    hipLaunchKernelGGL(rows_topk_kernel, dim3(T), dim3(256), 0, stream, lg, V, k, topk_id,
                       topk_logp, lse);
  } else {
    return EAGLE_EINVAL;
  }
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

// Scratch of eagle_lmhead_topk_noalloc: the library's own copy of what the
// caller's workspace holds for eagle_lmhead_topk.  Every GPU the library
// runs on holds one for the life of the process.  Host code never uses the
// array's name as an address: the per-device address comes from
// hipGetSymbolAddress with that device current.
__device__ __attribute__((aligned(256))) char lm_scratch[EAGLE_LMHEAD_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_lm_scratch_mu;
static char* g_lm_scratch[kMaxDevices] = {};

static int lm_scratch_ptr(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return EAGLE_EHIP;
  EAGLE_REQUIRE(dev >= 0 && dev < kMaxDevices, EAGLE_EUNSUPPORTED);
  if (stream) {   // the scratch found is the current device's: the stream must be on it
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return EAGLE_EHIP;
    EAGLE_REQUIRE((int)sd == dev, EAGLE_EINVAL);
  }
  std::lock_guard<std::mutex> lock(g_lm_scratch_mu);
  if (!g_lm_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(lm_scratch)) != hipSuccess || !ptr) return EAGLE_EHIP;
    g_lm_scratch[dev] = (char*)ptr;
  }
  *out = g_lm_scratch[dev];
  return EAGLE_OK;
}

}  // namespace eagle

extern "C" int eagle_lmhead_topk(const void* f, const void* W, int32_t T, int32_t d, int32_t V,
                                 int32_t k, eagle_dtype dt, const float* in_ssq, int32_t in_parts,
                                 float in_eps, int32_t* topk_id, float* topk_logp, float* lse,
                                 float* logits, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
  return eagle::lm_run(f, W, T, d, V, k, dt, in_ssq, in_parts, in_eps, topk_id, topk_logp, lse,
                       logits, (char*)workspace, ws_bytes, stream);
}

extern "C" int eagle_lmhead_topk_noalloc(const void* f, const void* W, int32_t T, int32_t d,
                                         int32_t V, int32_t k, eagle_dtype dt,
                                         const float* in_ssq, int32_t in_parts, float in_eps,
                                         int32_t* topk_id, float* topk_logp, float* lse,
                                         float* logits, hipStream_t stream) {
  using namespace eagle;
  // size first, so an oversized request fails before any HIP call
  EAGLE_REQUIRE(T >= 1 && V >= 1 && k >= 0, EAGLE_EINVAL);
  EAGLE_REQUIRE(dt == EAGLE_BF16 || dt == EAGLE_F32, EAGLE_EINVAL);
  EAGLE_REQUIRE(lm_layout(T, V, k, dt).total <= EAGLE_LMHEAD_SCRATCH_BYTES, EAGLE_EWORKSPACE);
  char* ws = nullptr;
  const int rc = lm_scratch_ptr(stream, &ws);
  if (rc != EAGLE_OK) return rc;
  return lm_run(f, W, T, d, V, k, dt, in_ssq, in_parts, in_eps, topk_id, topk_logp, lse, logits,
                ws, EAGLE_LMHEAD_SCRATCH_BYTES, stream);
}
