// Tree-masked attention of draft-tree nodes against a KV prefix.
//
// Sources: "EAGLE-2: Feature-Level Speculative Decoding Guide", Key
// Architectural Mechanics 3 - every tree node is scored in one batched pass
// under the tree mask (ancestors only); "Support Eagle-3 Speculative Decoding
// in llama.cpp" printout - grouped-query attention, 32 query / 8 KV heads of
// 128 dims.
//
// bf16 path, one workgroup = (KV head g, one slice of the positions, one group
// of 16 NTW NW query rows).  The query rows of a KV head are all (node i, head
// h) pairs with h / G = g, so every K/V tile fetched from HBM serves the G
// heads that share it (GQA) and all tree nodes at once.  The prefix is cut
// into splits of whole 64-position tiles; the tree is one more split, masked
// by the node's ancestor bits (64 tree positions per tile = one mask word).
// Each split writes unnormalised partials (row max, row sum, O) and a second
// kernel combines the splits (log-sum-exp merge).
//
// Per 64-position tile, per wave (16 NTW rows):
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, K from LDS as the A operand
//                 (positions = M), Q^T held in registers as the B operand;
//   online softmax in the exp2 domain (scale * log2 e folded into one FMA);
//   O^T += V^T P^T  with P^T taken straight from the S^T accumulators: a lane
//                 holds 4 consecutive positions of one query row per 16-row
//                 tile, so two tiles give the 8 k-values of a B operand once
//                 the k order is permuted.  V stays row-major in LDS (stored
//                 like K, 16 bytes per lane); its A operand is read with the
//                 gfx950 transposing LDS read ds_read_b64_tr_b16, which hands
//                 lane i of a 16-lane group element j of the 8-byte chunk that
//                 lane 4j + i/4 addressed (position i mod 4 of it): pointing
//                 lane (g, r16) at V[4g + r16/4][4 (r16 mod 4)] of a 16-dim
//                 slice gives it V[4g + j][r16] for j < 4, i.e. four positions
//                 of one head dim, in the permuted k order.
// K and V tiles are fetched two ahead into registers (16-byte buffer loads,
// coalesced along the head dimension) and double-buffered in LDS, one barrier
// per tile.  The loads are unconditional: positions past the slice fall
// outside the buffer range and read as zero without touching memory, so the
// number of loads in flight is fixed and the waits before each LDS store let
// the newer tile stay in flight.  The tree slice's mask words (at most four
// per row) are staged in LDS before the loop, behind the first K/V loads.
// The running max is raised lazily (see the softmax step).
//
// fp32 path (small workloads): one workgroup per (query row, head, split)
// computes the scores into LDS in fp32 and reduces them directly; same
// partial layout and merge.
#include "common.h"

namespace eagle {

constexpr int kAtTile = 64;
constexpr int kAtF32Chunk = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

struct AttnParams {
  const bf16_t* q;
  const bf16_t* kc;
  const bf16_t* vc;
  const bf16_t* kt;
  const bf16_t* vt;
  int64_t L, ldc;
  int Tk, ldt;
  const uint64_t* mask;
  int words, mask_rows;
  const int32_t* qmap;
  int Tq, Hq, Hkv, G;
  float c;               // scale * log2(e)
  int n_split;           // prefix splits; split index n_split is the tree
  int tiles_per_split;
  void* part_o;          // [n_split + 1][Tq * Hq][HD]: bf16 O / l (bf16 path), fp32 O (fp32 path)
  float2* part_ml;       // [n_split + 1][Tq * Hq] (running max, sum of weights)
  int32_t* status;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read of 4 bf16 (see the file comment for the lane layout).
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

// Online softmax of tile t's scores s (S^T accumulators: lane (g, r16) holds
// positions 16 mt + 4 g + j of query row 16 nt + r16) into bf16 weights pb
// (B operands of the V product), updating m, l and, when the running max
// moves, O.  ms: the wave's mask words per row tile and row (tree slice only).
template <int NTW, int MTV>
__device__ __forceinline__ void tile_softmax(int t, int npos, bool is_tree,
                                             const uint64_t (*ms)[16][4], float c, int g, int r16,
                                             f32x4 (&s)[4][NTW], u32x4 (&pb)[2][NTW],
                                             float (&m)[NTW], float (&l)[NTW],
                                             f32x4 (&o)[MTV][NTW]) {
  // visibility: positions past the slice end, and non-ancestors in the tree
  const int tile_pos = t * kAtTile;
  if (is_tree || tile_pos + kAtTile > npos) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      uint64_t bits = ~0ull;
      if (is_tree) bits = ms[nt][r16][t];  // t < words <= 4
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int pl = mt * 16 + 4 * g + j;
          if (tile_pos + pl >= npos || !((bits >> pl) & 1ull)) s[mt][nt][j] = -INFINITY;
        }
    }
  }

  // Online softmax in the exp2 domain with a lazily raised running max: m
  // only moves when the tile's max exceeds it by more than 2^8 (in exp2
  // units), so weights stay <= 2^8 and m, l and O always share the same
  // reference (exact); after the first tile the rescale is almost never
  // taken.  exp2 arguments are <= 8: the native v_exp_f32 is exact enough.
  float mx[NTW];
  bool up_any = false;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    float v = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) v = fmaxf(v, s[mt][nt][j]);
    mx[nt] = rows_max(v);
    up_any |= (mx[nt] - m[nt]) * c > 8.0f;
  }
  if (__builtin_amdgcn_ballot_w64(up_any)) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const bool up = (mx[nt] - m[nt]) * c > 8.0f;
      const float alpha = up ? __builtin_amdgcn_exp2f((m[nt] - mx[nt]) * c) : 1.0f;
      m[nt] = up ? mx[nt] : m[nt];
      l[nt] *= alpha;
#pragma unroll
      for (int mv = 0; mv < MTV; ++mv) o[mv][nt] *= alpha;
    }
  }
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const float nmc = -m[nt] * c;
    float ps = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[mt][nt][j], c, nmc));
        s[mt][nt][j] = pv;
        ps += pv;
      }
    l[nt] += ps;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      pb[kb2][nt] = u32x4{pack_bf16x2(s[2 * kb2][nt][0], s[2 * kb2][nt][1]),
                          pack_bf16x2(s[2 * kb2][nt][2], s[2 * kb2][nt][3]),
                          pack_bf16x2(s[2 * kb2 + 1][nt][0], s[2 * kb2 + 1][nt][1]),
                          pack_bf16x2(s[2 * kb2 + 1][nt][2], s[2 * kb2 + 1][nt][3])};
    }
  }
}

// Visibility of tile t's scores: positions past the slice end, and tree
// nodes that are not ancestors of the row's node, are set to -inf.
template <int NTW>
__device__ __forceinline__ void mask_scores(int t, int npos, bool is_tree,
                                            const uint64_t (*ms)[16][4], int g, int r16,
                                            f32x4 (&s)[4][NTW]) {
  const int tile_pos = t * kAtTile;
  if (is_tree || tile_pos + kAtTile > npos) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      uint64_t bits = ~0ull;
      if (is_tree) bits = ms[nt][r16][t];  // t < words <= 4
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int pl = mt * 16 + 4 * g + j;
          if (tile_pos + pl >= npos || !((bits >> pl) & 1ull)) s[mt][nt][j] = -INFINITY;
        }
    }
  }
}

// tile_softmax for scores that arrive already scaled by scale * log2(e) (q
// folded) and shifted: s = score - mi[row], the score MFMAs having started
// from -mi instead of 0.  m is the running max in the same scaled units.
// While m stays put and mi == m (every tile after a slice's first, almost
// always), the weights are exp2(s) with no arithmetic in between; a tile
// that raises m (or the first, where mi = 0) also subtracts m - mi.  On
// return mi = m, the offset for the next tile's score MFMAs.
template <int NTW, int MTV>
__device__ __forceinline__ void tile_softmax_shifted(int t, int npos, bool is_tree,
                                                     const uint64_t (*ms)[16][4], int g, int r16,
                                                     f32x4 (&s)[4][NTW], u32x4 (&pb)[2][NTW],
                                                     float (&m)[NTW], f32x4 (&ls)[NTW],
                                                     f32x4 (&o)[MTV][NTW], float (&mi)[NTW]) {
  mask_scores<NTW>(t, npos, is_tree, ms, g, r16, s);
  float mx[NTW];
  bool up_any = false, shift_any = false;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    float v = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) v = fmaxf(v, s[mt][nt][j]);
    mx[nt] = rows_max(v) + mi[nt];       // the tile's max score
    up_any |= mx[nt] - m[nt] > 8.0f;
    shift_any |= m[nt] != mi[nt];
  }
  if (__builtin_amdgcn_ballot_w64(up_any | shift_any)) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const bool up = mx[nt] - m[nt] > 8.0f;
      const float alpha = up ? __builtin_amdgcn_exp2f(m[nt] - mx[nt]) : 1.0f;
      m[nt] = up ? mx[nt] : m[nt];
      ls[nt] *= alpha;
#pragma unroll
      for (int mv = 0; mv < MTV; ++mv) o[mv][nt] *= alpha;
      const float d = m[nt] - mi[nt];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[mt][nt][j] -= d;
      mi[nt] = m[nt];
    }
  }
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[mt][nt][j] = __builtin_amdgcn_exp2f(s[mt][nt][j]);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      pb[kb2][nt] = u32x4{pack_bf16x2(s[2 * kb2][nt][0], s[2 * kb2][nt][1]),
                          pack_bf16x2(s[2 * kb2][nt][2], s[2 * kb2][nt][3]),
                          pack_bf16x2(s[2 * kb2 + 1][nt][0], s[2 * kb2 + 1][nt][1]),
                          pack_bf16x2(s[2 * kb2 + 1][nt][2], s[2 * kb2 + 1][nt][3])};
    }
  }
}

// (one 16-row tile per wave: registers for two workgroups per CU, so that a
// grid of a few hundred slices runs in one round)
template <int HD, int NTW, int NW>
__global__ __launch_bounds__(64 * NW, NTW == 1 ? 2 : 1) void tree_attn_bf16_kernel(AttnParams p) {
  constexpr int NTH = 64 * NW;
  constexpr int KB = HD / 32;
  constexpr int MTV = HD / 16;
  // row strides: K rows 8 elements past a bank round (16 lanes of a b128 read
  // on distinct banks), V rows 16 past (the four rows a 16-lane group reads
  // with the transposing b64 read on disjoint banks)
  constexpr int KS = HD + 8;
  constexpr int VS = HD + 16;
  constexpr int CPR = HD / 8;
  constexpr int NCH = kAtTile * CPR / NTH;
  // K and V double buffers; after the last tile the same space stages each
  // wave's output rows (PS bytes apart) for row-contiguous stores
  constexpr int PS = HD * 2 + 16;
  constexpr int SMEM = 2 * kAtTile * (KS + VS);
  static_assert(NW * 16 * NTW * PS <= SMEM * 2, "output staging fits the K/V buffers");
  __shared__ __attribute__((aligned(16))) bf16_t smem[SMEM];
  bf16_t(*Ks)[kAtTile * KS] = (bf16_t(*)[kAtTile * KS])smem;
  bf16_t(*Vs)[kAtTile * VS] = (bf16_t(*)[kAtTile * VS])(smem + 2 * kAtTile * KS);
  __shared__ uint64_t Ms[NW][NTW][16][4];  // tree slice: each row's mask words

  const int split = blockIdx.x;
  const int gkv = blockIdx.y;
  const int qg = blockIdx.z;
  const bool is_tree = split == p.n_split;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int R = p.Tq * p.G;
  const int RT = p.Tq * p.Hq;

  int grow[NTW];
  bool valid[NTW];
  int mrow[NTW];
  u32x4 qf[NTW][KB];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int r = qg * (16 * NTW * NW) + wave * 16 * NTW + nt * 16 + r16;
    valid[nt] = r < R;
    const int i = valid[nt] ? r / p.G : 0;
    const int h = gkv * p.G + (valid[nt] ? r % p.G : 0);
    grow[nt] = i * p.Hq + h;
    mrow[nt] = is_tree ? (p.qmap ? p.qmap[i] : i) : 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qf[nt][kb] = valid[nt] ? *(const u32x4*)(p.q + (size_t)grow[nt] * HD + kb * 32 + 8 * g)
                             : u32x4{0u, 0u, 0u, 0u};
  }

  int64_t pos0;
  int npos;
  const bf16_t* kb_ptr;
  const bf16_t* vb_ptr;
  if (!is_tree) {
    pos0 = (int64_t)split * p.tiles_per_split * kAtTile;
    const int64_t rest = p.L - pos0;
    npos = rest > (int64_t)p.tiles_per_split * kAtTile ? p.tiles_per_split * kAtTile : (int)rest;
    kb_ptr = p.kc + ((size_t)gkv * p.ldc + pos0) * HD;
    vb_ptr = p.vc + ((size_t)gkv * p.ldc + pos0) * HD;
  } else {
    pos0 = 0;
    npos = p.Tk;
    kb_ptr = p.kt + (size_t)gkv * p.ldt * HD;
    vb_ptr = p.vt + (size_t)gkv * p.ldt * HD;
  }
  const int ntiles = npos > 0 ? (npos + kAtTile - 1) / kAtTile : 0;

  float m[NTW], l[NTW];
  f32x4 o[MTV][NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    m[nt] = kNegBig;
    l[nt] = 0.f;
#pragma unroll
    for (int mv = 0; mv < MTV; ++mv) o[mv][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // K/V tiles go HBM -> registers (two stages: up to two tiles in flight, each
  // with two tile-times to arrive) -> LDS (two buffers: one barrier per tile).
  const __amdgpu_buffer_rsrc_t krs = buf_rsrc(kb_ptr, (size_t)npos * HD * sizeof(bf16_t));
  const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(vb_ptr, (size_t)npos * HD * sizeof(bf16_t));
  u32x4 kr0[NCH], vr0[NCH], kr1[NCH], vr1[NCH];
  auto load_tile = [&](int t, u32x4 (&kr)[NCH], u32x4 (&vr)[NCH]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      // chunk c = tid + NTH j of the tile: position c / CPR, 8 dims at (c mod CPR) 8
      const uint32_t off = (uint32_t)(t * kAtTile * HD + (tid + NTH * j) * 8) * sizeof(bf16_t);
      kr[j] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
      vr[j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
    }
  };
  auto store_tile = [&](int buf, const u32x4 (&kr)[NCH], const u32x4 (&vr)[NCH])
                        __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = tid + NTH * j;
      const int pr = c / CPR;
      const int cc = c - pr * CPR;
      *(u32x4*)(&Ks[buf][pr * KS + cc * 8]) = kr[j];
      *(u32x4*)(&Vs[buf][pr * VS + cc * 8]) = vr[j];
    }
  };

  // S^T = K Q^T over the 4 position tiles of 16 of LDS buffer `buf`
  auto qk = [&](int buf, f32x4 (&s)[4][NTW]) __attribute__((always_inline)) {
    const bf16_t* Kb = Ks[buf];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) s[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = *(const bf16x8*)(&Kb[(mt * 16 + r16) * KS + kb * 32 + 8 * g]);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(qf[nt][kb]),
                                                              s[mt][nt], 0, 0, 0);
      }
    }
  };

  auto softmax = [&](int t, f32x4 (&s)[4][NTW], u32x4 (&pb)[2][NTW])
                     __attribute__((always_inline)) {
    tile_softmax<NTW, MTV>(t, npos, is_tree, Ms[wave], p.c, g, r16, s, pb, m, l, o);
  };

  // O^T += V^T P^T from LDS buffer `buf`
  auto pv = [&](int buf, const u32x4 (&pb)[2][NTW]) __attribute__((always_inline)) {
    const bf16_t* Vb = Vs[buf];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int mv = 0; mv < MTV; ++mv) {
        // k slots 0-3: positions 32 kb2 + 4 g + j; slots 4-7: 16 further
        const bf16_t* vp = &Vb[(kb2 * 32 + 4 * g + (r16 >> 2)) * VS + mv * 16 + 4 * (r16 & 3)];
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi = lds_read_tr16(vp + 16 * VS);
        const bf16x8 a = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          o[mv][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(pb[kb2][nt]),
                                                              o[mv][nt], 0, 0, 0);
      }
    }
  };

  // One whole 64-position tile from LDS buffer `buf`.
  auto tile = [&](int t, int buf) __attribute__((always_inline)) {
    f32x4 s[4][NTW];
    u32x4 pb[2][NTW];
    qk(buf, s);
    softmax(t, s, pb);
    pv(buf, pb);
  };

  auto run_tiles = [&]() __attribute__((always_inline)) {
    if (ntiles == 0) return;
    // issue order fixed (tile 0, 1, 2) so that the waits before each store
    // count the same loads here as in the loop
    load_tile(0, kr0, vr0);
    __builtin_amdgcn_sched_barrier(0);
    load_tile(1, kr1, vr1);
    __builtin_amdgcn_sched_barrier(0);
    store_tile(0, kr0, vr0);
    load_tile(2, kr0, vr0);
    if (is_tree && g == 0) {
      // mask words of each row into LDS, read after the first K/V loads are
      // on their way
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int mr = mrow[nt];
        const bool ok = mr >= 0 && mr < p.mask_rows;
        if (valid[nt] && !ok) set_status(p.status, EAGLE_DEV_BAD_INDEX);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          Ms[wave][nt][r16][w] = ok && w < p.words ? p.mask[(size_t)mr * p.words + w] : 0ull;
      }
    }
    __syncthreads();
    // Loads past the last tile read zeros (out of the buffer range), so the
    // loop issues the same loads every iteration.  Single-exit loop with the
    // odd tile peeled: with an exit in the middle, the compiler waits for all
    // loads (the newer tile too) before the first store of each iteration.
    int t = 0;
#pragma clang loop unroll(disable)
    for (; t + 1 < ntiles; t += 2) {
      tile(t, 0);
      store_tile(1, kr1, vr1);
      load_tile(t + 3, kr1, vr1);
      __syncthreads();
      tile(t + 1, 1);
      if (t + 2 < ntiles) store_tile(0, kr0, vr0);  // (no wait for loads past the end)
      load_tile(t + 4, kr0, vr0);
      __syncthreads();
    }
    if (t < ntiles) tile(t, 0);
  };

  run_tiles();

  // Partials: O / l in bf16 (a convex combination of V rows: V's range, and a
  // rounding of 2^-9 relative, below the output's own bf16 rounding) and
  // (m, l).  Lane (g, r16) holds O^T[hd = 16 mv + 4 g + j][row 16 nt + r16]:
  // staged in LDS, then stored as whole rows, 16 bytes per lane (4 query heads
  // of one node are 4 consecutive rows in memory).
  __syncthreads();  // every wave is done with the K/V buffers
  char* stg = (char*)smem + wave * (16 * NTW) * PS;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const float lt = rows_sum(l[nt]);
    if (valid[nt] && g == 0) p.part_ml[(size_t)split * RT + grow[nt]] = make_float2(m[nt], lt);
    const float il = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
    for (int mv = 0; mv < MTV; ++mv) {
      const f32x4 v = o[mv][nt] * il;
      *(u32x2*)(stg + (nt * 16 + r16) * PS + (mv * 16 + 4 * g) * 2) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
  constexpr int CH = HD * 2 / 16;  // 16-byte chunks per row
#pragma unroll
  for (int k = 0; k < 16 * NTW * CH / 64; ++k) {
    const int idx = k * 64 + lane;
    const int rr = idx / CH;
    const int ch = idx - rr * CH;
    const int r = qg * (16 * NTW * NW) + wave * 16 * NTW + rr;
    if (r < R) {
      const int orow = (r / p.G) * p.Hq + gkv * p.G + r % p.G;
      *(u32x4*)((char*)p.part_o + ((size_t)split * RT + orow) * HD * 2 + ch * 16) =
          *(const u32x4*)(stg + rr * PS + ch * 16);
    }
  }
}

// Ring variant for 128-dim heads.  K/V tiles go straight from HBM into LDS
// (gfx950 16-byte buffer loads with an LDS destination) through NST stages,
// so NST - 1 tiles are in flight while one is computed, and no registers
// stage them.  A load instruction fills 1 KB of LDS contiguously (lane l at
// byte 16 l), so rows cannot be padded; instead 16-byte chunk c of row r is
// stored at chunk c ^ (r mod 16) for K (the 16 rows one b128 read touches fall
// on distinct banks) and at c ^ 2 (r mod 8) for V (the 8 rows of a 32-lane
// half of a transposing read keep their 32-byte column pair whole and apart).
// The stages are separate LDS objects, so the compiler's own wait before an
// LDS read covers only the loads into that stage.  Each step waits for the
// wave's own loads of the current tile; the barrier that follows publishes
// every wave's part and tells all waves that the stage about to be refilled
// is no longer read.  Compute per tile is that of tree_attn_bf16_kernel.
constexpr int kRingHD = 128;
constexpr int kRingTileBytes = kAtTile * kRingHD * 2;  // one K (or V) tile: 16 KB

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from the buffer at byte offset off into LDS at
// lds + 16 lane (lds is the same for the whole wave).  The host pass has no
// such builtin and never runs this.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, bf16_t* lds, uint32_t off) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, off, 0, 0, 0);
#endif
}

template <int NTW, int NW, int NST>
__global__ __launch_bounds__(64 * NW, 1) void tree_attn_ring_kernel(AttnParams p) {
  constexpr int HD = kRingHD;
  constexpr int KB = HD / 32;
  constexpr int MTV = HD / 16;
  constexpr int TB = kRingTileBytes;
  constexpr int IPT = TB / 1024 / NW;  // 1 KB load instructions per thread per tile, K and V each
  constexpr int PS = HD * 2 + 16;      // output staging row stride (bytes)
  static_assert(NST >= 2 && NST <= 4 && IPT >= 1 && TB % (1024 * NW) == 0, "ring shape");
  static_assert(NW <= 2 * NST && 16 * NTW * PS <= TB, "output staging: half a stage per wave");
  // stage s: K tile at [0, TB), V tile at [TB, 2 TB)
  __shared__ __attribute__((aligned(1024))) bf16_t st0[2 * kAtTile * HD];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[2 * kAtTile * HD];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[NST > 2 ? 2 * kAtTile * HD : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[NST > 3 ? 2 * kAtTile * HD : 8];
  __shared__ uint64_t Ms[NW][NTW][16][4];  // tree slice: each row's mask words

  const int split = blockIdx.x;
  const int gkv = blockIdx.y;
  const int qg = blockIdx.z;
  const bool is_tree = split == p.n_split;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int R = p.Tq * p.G;
  const int RT = p.Tq * p.Hq;

  int grow[NTW];
  bool valid[NTW];
  int mrow[NTW];
  u32x4 qf[NTW][KB];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int r = qg * (16 * NTW * NW) + wave * 16 * NTW + nt * 16 + r16;
    valid[nt] = r < R;
    const int i = valid[nt] ? r / p.G : 0;
    const int h = gkv * p.G + (valid[nt] ? r % p.G : 0);
    grow[nt] = i * p.Hq + h;
    mrow[nt] = is_tree ? (p.qmap ? p.qmap[i] : i) : 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qf[nt][kb] = valid[nt] ? *(const u32x4*)(p.q + (size_t)grow[nt] * HD + kb * 32 + 8 * g)
                             : u32x4{0u, 0u, 0u, 0u};
  }
  // scale * log2(e) folded into q once (one more bf16 rounding, 2^-9
  // relative): the score MFMAs then deliver exp2 arguments directly
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = qf[nt][kb][e];
        qf[nt][kb][e] = pack_bf16x2(bf16_bits_to_f32(w & 0xffffu) * p.c, bf16_bits_to_f32(w >> 16) * p.c);
      }

  int64_t pos0;
  int npos;
  const bf16_t* kb_ptr;
  const bf16_t* vb_ptr;
  if (!is_tree) {
    pos0 = (int64_t)split * p.tiles_per_split * kAtTile;
    const int64_t rest = p.L - pos0;
    npos = rest > (int64_t)p.tiles_per_split * kAtTile ? p.tiles_per_split * kAtTile : (int)rest;
    kb_ptr = p.kc + ((size_t)gkv * p.ldc + pos0) * HD;
    vb_ptr = p.vc + ((size_t)gkv * p.ldc + pos0) * HD;
  } else {
    pos0 = 0;
    npos = p.Tk;
    kb_ptr = p.kt + (size_t)gkv * p.ldt * HD;
    vb_ptr = p.vt + (size_t)gkv * p.ldt * HD;
  }
  const int ntiles = npos > 0 ? (npos + kAtTile - 1) / kAtTile : 0;

  // m: running max of the scaled scores; mi: the offset the score MFMAs start
  // from (-mi in every accumulator), 0 until the first tile sets m
  float m[NTW], mi[NTW];
  f32x4 o[MTV][NTW], ls[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    m[nt] = kNegBig;
    ls[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mi[nt] = 0.f;
#pragma unroll
    for (int mv = 0; mv < MTV; ++mv) o[mv][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // This thread's chunks of a tile: instruction j of wave w fills LDS chunks
  // 64 b .. 64 b + 63 (b = j NW + w), i.e. rows 4 b .. 4 b + 3; lane l takes
  // row 4 b + l / 16, LDS chunk l mod 16, and loads the chunk of the row that
  // the swizzle puts there.  Byte offsets within tile 0 of the slice.
  const __amdgpu_buffer_rsrc_t krs = buf_rsrc(kb_ptr, (size_t)npos * HD * sizeof(bf16_t));
  const __amdgpu_buffer_rsrc_t vrs = buf_rsrc(vb_ptr, (size_t)npos * HD * sizeof(bf16_t));
  uint32_t koff[IPT], voff[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int r = 4 * (j * NW + wave) + (lane >> 4);
    const int cl = lane & 15;
    koff[j] = (uint32_t)(r * 256 + ((cl ^ (r & 15)) << 4));
    voff[j] = (uint32_t)(r * 256 + ((cl ^ (2 * (r & 7))) << 4));
  }
  // LDS read offsets (bytes): K chunk kb 4 + g of row 16 mt + r16; V as the
  // transposing read of tree_attn_bf16_kernel addresses it, swizzled
  uint32_t kro[KB], vro[MTV];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    kro[kb] = (uint32_t)(r16 * 256 + ((((kb ^ (r16 >> 2)) << 2) | (g ^ (r16 & 3))) << 4));
  const int pe = ((g & 1) << 2) | (r16 >> 2);  // row mod 8 of this lane's V rows
#pragma unroll
  for (int mv = 0; mv < MTV; ++mv)
    vro[mv] = (uint32_t)((4 * g + (r16 >> 2)) * 256 + 8 * (r16 & 3) + 32 * (mv ^ pe));

  auto stage = [&](int s) __attribute__((always_inline)) -> bf16_t* {
    // s is a compile-time constant at every call (unrolled steps)
    return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3;
  };
  auto issue = [&](int t, bf16_t* stg) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)t * TB;
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      lds_load16(krs, stg + (j * NW + wave) * 512, base + koff[j]);
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      lds_load16(vrs, stg + kAtTile * HD + (j * NW + wave) * 512, base + voff[j]);
  };

  auto qk = [&](const bf16_t* stg, f32x4 (&s)[4][NTW]) __attribute__((always_inline)) {
    f32x4 c0[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) c0[nt] = f32x4{-mi[nt], -mi[nt], -mi[nt], -mi[nt]};
    const char* Kb = (const char*)stg;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = *(const bf16x8*)(Kb + mt * 4096 + kro[kb]);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, as_bf16x8(qf[nt][kb]), kb == 0 ? c0[nt] : s[mt][nt], 0, 0, 0);
      }
    }
  };
  auto pv = [&](const bf16_t* stg, const u32x4 (&pb)[2][NTW]) __attribute__((always_inline)) {
    const char* Vb = (const char*)(stg + kAtTile * HD);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int mv = 0; mv < MTV; ++mv) {
        const u32x2 lo = lds_read_tr16((const bf16_t*)(Vb + kb2 * 8192 + vro[mv]));
        const u32x2 hi = lds_read_tr16((const bf16_t*)(Vb + kb2 * 8192 + 4096 + vro[mv]));
        const bf16x8 a = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          o[mv][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(pb[kb2][nt]),
                                                              o[mv][nt], 0, 0, 0);
      }
      // row sums of the weights: every row of an all-ones A operand
      const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
        ls[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, as_bf16x8(pb[kb2][nt]), ls[nt], 0,
                                                         0, 0);
    }
  };
  auto step = [&](int t, int s) __attribute__((always_inline)) {
    // this wave's loads of tile t are done (the NST - 2 newer tiles may still
    // be in flight), then every wave's are, and stage s - 1 is free
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((NST - 2) * 2 * IPT, 0));
    asm volatile("s_barrier" ::: "memory");
    issue(t + NST - 1, stage((s + NST - 1) % NST));
    if (t < ntiles) {
      f32x4 sc[4][NTW];
      u32x4 pb[2][NTW];
      qk(stage(s), sc);
      tile_softmax_shifted<NTW, MTV>(t, npos, is_tree, Ms[wave], g, r16, sc, pb, m, ls, o, mi);
      pv(stage(s), pb);
    }
  };

  if (ntiles > 0) {
    issue(0, st0);
    if (NST > 2) issue(1, st1);
    if (NST > 3) issue(2, st2);
    if (is_tree && g == 0) {
      // mask words of each row into LDS, behind the first K/V loads
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int mr = mrow[nt];
        const bool ok = mr >= 0 && mr < p.mask_rows;
        if (valid[nt] && !ok) set_status(p.status, EAGLE_DEV_BAD_INDEX);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          Ms[wave][nt][r16][w] = ok && w < p.words ? p.mask[(size_t)mr * p.words + w] : 0ull;
      }
    }
    // Whole rounds of NST steps; steps past the last tile only keep the
    // barrier and load counts uniform (their loads fall outside the buffer
    // range and read zero without touching memory).
#pragma clang loop unroll(disable)
    for (int t0 = 0; t0 < ntiles; t0 += NST) {
      step(t0, 0);
      step(t0 + 1, 1);
      if (NST > 2) step(t0 + 2, 2);
      if (NST > 3) step(t0 + 3, 3);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  }

  // Partials, as in tree_attn_bf16_kernel: O / l in bf16 and (m, l), O rows
  // staged in LDS (half a stage per wave) and stored as whole rows.
  __syncthreads();  // every wave is done with the stages and no load is in flight
  char* stg = (char*)stage(wave >> 1) + (wave & 1) * TB;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const float lt = ls[nt][0];          // (the four values of a lane are the same sum)
    // (m back in score units for the merge, which scales by scale * log2(e))
    if (valid[nt] && g == 0)
      p.part_ml[(size_t)split * RT + grow[nt]] = make_float2(m[nt] / p.c, lt);
    const float il = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
    for (int mv = 0; mv < MTV; ++mv) {
      const f32x4 v = o[mv][nt] * il;
      *(u32x2*)(stg + (nt * 16 + r16) * PS + (mv * 16 + 4 * g) * 2) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
  constexpr int CH = HD * 2 / 16;  // 16-byte chunks per row
#pragma unroll
  for (int k = 0; k < 16 * NTW * CH / 64; ++k) {
    const int idx = k * 64 + lane;
    const int rr = idx / CH;
    const int ch = idx - rr * CH;
    const int r = qg * (16 * NTW * NW) + wave * 16 * NTW + rr;
    if (r < R) {
      const int orow = (r / p.G) * p.Hq + gkv * p.G + r % p.G;
      *(u32x4*)((char*)p.part_o + ((size_t)split * RT + orow) * HD * 2 + ch * 16) =
          *(const u32x4*)(stg + rr * PS + ch * 16);
    }
  }
}

// fp32 path: one workgroup per (split, query row, head).
__global__ __launch_bounds__(256) void tree_attn_f32_kernel(AttnParams p, int hd) {
  __shared__ float sc[kAtF32Chunk];
  __shared__ float qs[256];
  __shared__ float red[4];
  const int split = blockIdx.x;
  const int grow = blockIdx.y;
  const bool is_tree = split == p.n_split;
  const int i = grow / p.Hq;
  const int h = grow - i * p.Hq;
  const int gkv = h / p.G;
  const float* q = (const float*)p.q;
  const int RT = p.Tq * p.Hq;
  for (int d = threadIdx.x; d < hd; d += 256) qs[d] = q[(size_t)grow * hd + d];
  int64_t pos0, npos;
  const float* kp;
  const float* vp;
  int mr = -1;
  if (!is_tree) {
    pos0 = (int64_t)split * kAtF32Chunk;
    npos = p.L - pos0;
    if (npos > kAtF32Chunk) npos = kAtF32Chunk;
    kp = (const float*)p.kc + ((size_t)gkv * p.ldc + pos0) * hd;
    vp = (const float*)p.vc + ((size_t)gkv * p.ldc + pos0) * hd;
  } else {
    pos0 = 0;
    npos = p.Tk;
    kp = (const float*)p.kt + (size_t)gkv * p.ldt * hd;
    vp = (const float*)p.vt + (size_t)gkv * p.ldt * hd;
    mr = p.qmap ? p.qmap[i] : i;
    if (mr < 0 || mr >= p.mask_rows) {
      if (threadIdx.x == 0 && h == 0) set_status(p.status, EAGLE_DEV_BAD_INDEX);
      mr = -1;
    }
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < npos; j += 256) {
    bool vis = true;
    if (is_tree) vis = mr >= 0 && ((p.mask[(size_t)mr * p.words + (j >> 6)] >> (j & 63)) & 1ull);
    float s = -INFINITY;
    if (vis) {
      s = 0.f;
      const float* kr = kp + (size_t)j * hd;
      for (int d = 0; d < hd; ++d) s = fmaf(qs[d], kr[d], s);
    }
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), kNegBig);
  float ls = 0.f;
  for (int j = threadIdx.x; j < npos; j += 256) {
    const float pv = exp2f((sc[j] - M) * p.c);
    sc[j] = pv;
    ls += pv;
  }
  ls = wave_sum(ls);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ls;
  __syncthreads();
  const float lt = ((red[0] + red[1]) + red[2]) + red[3];
  const size_t prow = (size_t)split * RT + grow;
  for (int d = threadIdx.x; d < hd; d += 256) {
    float a = 0.f;
    for (int j = 0; j < npos; ++j) a = fmaf(sc[j], vp[(size_t)j * hd + d], a);
    ((float*)p.part_o)[prow * hd + d] = a;
  }
  if (threadIdx.x == 0) p.part_ml[prow] = make_float2(M, lt);
}

// Combine the splits of each (query row, head).  With w_s = 2^((m_s - M) c)
// and M = max_s m_s: out = sum_s w_s O_s / sum_s w_s l_s.  The bf16 path
// stores o_s = O_s / l_s (so O_s = l_s o_s), the fp32 path O_s itself.
constexpr int kMergeSplits = 1024;

// bf16 partials.  One block of four waves per RPW consecutive rows (4 rows
// of 128 dims, 8 of 64).  Lane (row rr, chunk ch) of wave v sums 8 head dims
// of its row over the splits s = v, v + 4, v + 8, ... in ascending order,
// one 16-byte load per split; its first LPB loads are issued before anything
// else, so their latency overlaps the split weights l_s w_s, which wave q
// forms for rows q, q + 4, ... (lanes over splits) into LDS.  Wave 0 then
// adds the other waves' sums in wave order and writes the row.  The weights
// take RPW * nsplit floats of dynamic LDS and the kernel ~108 registers, so
// four blocks share a CU.
template <int HD>
__global__ __launch_bounds__(256) void attn_merge_bf16_kernel(const bf16_t* __restrict__ part_o,
                                                              const float2* __restrict__ part_ml,
                                                              int nsplit, int RT, float c,
                                                              void* out, int out_bf16) {
  constexpr int CPR = HD / 8;    // 16-byte chunks per row
  constexpr int RPW = 64 / CPR;  // rows per block
  constexpr int NWV = 4;         // waves per block
  constexpr int LPB = 8;         // loads in flight per lane
  extern __shared__ float wsh[];  // [RPW][nsplit]
  __shared__ float dsh[RPW];
  __shared__ f32x4 accs[NWV - 1][2][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row0 = blockIdx.x * RPW;
  const int rr = lane / CPR;
  const int ch = lane - rr * CPR;
  const int row = row0 + rr;
  const bool live = row < RT;
  const bf16_t* po = part_o + (size_t)(live ? row : 0) * HD + ch * 8;
  const size_t stride = (size_t)RT * HD;
  auto load_batch = [&](int s0, u32x4 (&v)[LPB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LPB; ++u) {
      const int s = s0 + NWV * u;
      v[u] = (live && s < nsplit) ? *(const u32x4*)(po + (size_t)s * stride)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 v[LPB];
  load_batch(wave, v);

  for (int q = wave; q < RPW; q += NWV) {
    const int r = row0 + q;
    float M = kNegBig;
    if (r < RT)
      for (int s = lane; s < nsplit; s += 64) M = fmaxf(M, part_ml[(size_t)s * RT + r].x);
    M = wave_max(M);
    float den = 0.f;
    if (r < RT)
      for (int s = lane; s < nsplit; s += 64) {
        const float2 ml = part_ml[(size_t)s * RT + r];
        const float w = exp2f((ml.x - M) * c) * ml.y;
        wsh[q * nsplit + s] = w;
        den += w;
      }
    den = wave_sum(den);
    if (lane == 0) dsh[q] = den;
  }
  __syncthreads();
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s0 = wave;;) {
#pragma unroll
    for (int u = 0; u < LPB; ++u) {
      const int s = s0 + NWV * u;
      const float w = s < nsplit ? wsh[rr * nsplit + s] : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(__uint_as_float(v[u][e] << 16), w, acc[2 * e]);
        acc[2 * e + 1] = fmaf(__uint_as_float(v[u][e] & 0xffff0000u), w, acc[2 * e + 1]);
      }
    }
    s0 += NWV * LPB;
    if (s0 >= nsplit) break;
    load_batch(s0, v);
  }
  if (wave > 0) {
    accs[wave - 1][0][lane] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    accs[wave - 1][1][lane] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
  __syncthreads();
  if (wave != 0 || !live) return;
#pragma unroll
  for (int w = 0; w < NWV - 1; ++w) {
    const f32x4 a = accs[w][0][lane];
    const f32x4 b = accs[w][1][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += a[e];
      acc[4 + e] += b[e];
    }
  }
  const float dsel = dsh[rr];
  const float inv = dsel > 0.f ? 1.0f / dsel : 0.f;
  if (out_bf16) {
    *(u32x4*)((bf16_t*)out + (size_t)row * HD + ch * 8) =
        u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
              pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  } else {
    float* o = (float*)out + (size_t)row * HD + ch * 8;
    *(f32x4*)o = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *(f32x4*)(o + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
}

// fp32 partials (O_s unnormalised), one block per output row: the split
// weights are formed once per row in LDS; each thread then sums one head-dim
// element over the splits.
__global__ __launch_bounds__(128) void attn_merge_f32_kernel(const float* __restrict__ part_o,
                                                             const float2* __restrict__ part_ml,
                                                             int nsplit, int RT, int hd, float c,
                                                             void* out, int out_bf16) {
  __shared__ float wsh[kMergeSplits];
  __shared__ float red[2];
  const int row = blockIdx.x;
  float M = kNegBig;
  for (int s = threadIdx.x; s < nsplit; s += blockDim.x)
    M = fmaxf(M, part_ml[(size_t)s * RT + row].x);
  M = wave_max(M);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  for (int s = threadIdx.x; s < nsplit; s += blockDim.x)
    wsh[s] = exp2f((part_ml[(size_t)s * RT + row].x - M) * c);
  __syncthreads();
  float den = 0.f;
  for (int s = 0; s < nsplit; ++s) den = fmaf(part_ml[(size_t)s * RT + row].y, wsh[s], den);
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  for (int d = threadIdx.x; d < hd; d += blockDim.x) {
    float num = 0.f;
    const float* po = part_o + (size_t)row * hd + d;
#pragma unroll 4
    for (int s = 0; s < nsplit; ++s) num = fmaf(po[(size_t)s * RT * hd], wsh[s], num);
    const float v = num * inv;
    if (out_bf16)
      ((bf16_t*)out)[(size_t)row * hd + d] = (bf16_t)f32_to_bf16_bits(v);
    else
      ((float*)out)[(size_t)row * hd + d] = v;
  }
}

// ---------------------------------------------------------------- host side

struct AttnPlan {
  int ntw, nw, qgroups, n_split, tiles_per_split;
  size_t o_off, ml_off, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int64_t kCUs = 256;  // MI355X compute units

// The LDS-ring kernel serves 128-dim heads with 256 query rows per workgroup.
static bool ring_path(int hd, int nw) { return hd == kRingHD && nw == 8; }
constexpr int64_t kRingSliceOverhead = 3;

static AttnPlan attn_plan(int Tq, int Hq, int Hkv, int hd, int64_t L, eagle_dtype dt) {
  AttnPlan pl{};
  const int G = Hq / Hkv;
  const int R = Tq * G;
  if (dt == EAGLE_BF16) {
    // rows per workgroup: 64 (4 waves x 16), 128 (4 x 32) or 256 (8 x 32)
    pl.ntw = R <= 64 ? 1 : 2;
    pl.nw = R <= 128 ? 4 : 8;
    const int rows = 16 * pl.ntw * pl.nw;
    pl.qgroups = (R + rows - 1) / rows;
    const int64_t tiles = (L + kAtTile - 1) / kAtTile;
    if (tiles == 0) {
      pl.n_split = 0;
      pl.tiles_per_split = 1;
    } else if (ring_path(hd, pl.nw)) {
      // One workgroup per CU (the LDS ring): pick the slice length whose
      // grid (prefix slices plus the tree slice) needs the fewest tile-times,
      // counting whole rounds of kCUs workgroups and, per workgroup, the fixed
      // cost of loading its query rows and storing its partials (about
      // kRingSliceOverhead tile-times; without it one-tile slices win at 1024
      // rows per KV head and the partials outgrow the K/V); ties go to fewer
      // slices.
      const int64_t per_split_blocks = (int64_t)Hkv * pl.qgroups;
      const int64_t tps_min = (tiles + kMergeSplits - 2) / (kMergeSplits - 1);
      int64_t best_cost = -1;
      pl.tiles_per_split = (int)(tps_min < 65537 ? tps_min : 65537);  // (host checks reject > 65536)
      pl.n_split = (int)((tiles + pl.tiles_per_split - 1) / pl.tiles_per_split);
      for (int64_t tps = tps_min; tps <= tiles && tps <= 65536 && tps < tps_min + 4096; ++tps) {
        const int64_t n = (tiles + tps - 1) / tps;
        if (n + 1 > kMergeSplits) continue;
        const int64_t rounds = ((n + 1) * per_split_blocks + kCUs - 1) / kCUs;
        const int64_t cost = rounds * (tps + kRingSliceOverhead);
        if (best_cost < 0 || cost <= best_cost) {
          best_cost = cost;
          pl.tiles_per_split = (int)tps;
          pl.n_split = (int)n;
        }
      }
    } else {
      const int64_t per_split_blocks = (int64_t)Hkv * pl.qgroups;
      int64_t want = (256 + per_split_blocks - 1) / per_split_blocks;
      if (want < 1) want = 1;
      if (want > tiles) want = tiles;
      pl.tiles_per_split = (int)((tiles + want - 1) / want);
      pl.n_split = (int)((tiles + pl.tiles_per_split - 1) / pl.tiles_per_split);
    }
  } else {
    pl.ntw = 0;
    pl.nw = 4;
    pl.qgroups = 1;
    pl.n_split = (int)((L + kAtF32Chunk - 1) / kAtF32Chunk);
    pl.tiles_per_split = 0;
  }
  const size_t RT = (size_t)Tq * Hq;
  const size_t ns = (size_t)pl.n_split + 1;
  pl.o_off = 0;
  pl.ml_off = align256(ns * RT * hd * (dt == EAGLE_BF16 ? sizeof(bf16_t) : sizeof(float)));
  pl.total = pl.ml_off + align256(ns * RT * sizeof(float2));
  return pl;
}

template <int HD, int NTW, int NW>
static void launch_attn(const AttnParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((tree_attn_bf16_kernel<HD, NTW, NW>), grid, dim3(64 * NW), 0, s, p);
}

template <int NTW, int NW, int NST>
static void launch_ring(const AttnParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((tree_attn_ring_kernel<NTW, NW, NST>), grid, dim3(64 * NW), 0, s, p);
}

}  // namespace eagle

extern "C" size_t eagle_tree_attn_workspace(int32_t Tq, int32_t Hq, int32_t Hkv, int32_t hd,
                                            int64_t L, int32_t Tk, eagle_dtype in_dt) {
  (void)Tk;
  if (Tq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || hd < 1 || L < 0) return 0;
  return eagle::attn_plan(Tq, Hq, Hkv, hd, L, in_dt).total;
}

extern "C" int eagle_tree_attn(const void* q, const void* k_cache, const void* v_cache, int64_t L,
                               int64_t ld_cache, const void* k_tree, const void* v_tree,
                               int32_t Tk, int32_t ld_tree, const uint64_t* mask, int32_t words,
                               int32_t mask_rows, const int32_t* q_mask_row, int32_t Tq,
                               int32_t Hq, int32_t Hkv, int32_t hd, float scale,
                               eagle_dtype in_dt, eagle_dtype out_dt, void* out, void* workspace,
                               size_t ws_bytes, int32_t* dev_status, hipStream_t stream) {
  using namespace eagle;
  EAGLE_REQUIRE(q && k_tree && v_tree && mask && out && workspace, EAGLE_EINVAL);
  EAGLE_REQUIRE(L >= 0 && (L == 0 || (k_cache && v_cache && ld_cache >= L)), EAGLE_EINVAL);
  EAGLE_REQUIRE(Tq >= 1 && Tq <= EAGLE_MAX_TREE && Tk >= 1 && Tk <= EAGLE_MAX_TREE, EAGLE_EINVAL);
  EAGLE_REQUIRE(ld_tree >= Tk && words >= (Tk + 63) / 64 && words <= 4 && mask_rows >= 1,
                EAGLE_EINVAL);
  EAGLE_REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, EAGLE_EINVAL);
  EAGLE_REQUIRE(scale > 0.0f && scale < 3.0e38f, EAGLE_EINVAL);
  EAGLE_REQUIRE(in_dt == EAGLE_BF16 || in_dt == EAGLE_F32, EAGLE_EINVAL);
  EAGLE_REQUIRE(out_dt == EAGLE_BF16 || out_dt == EAGLE_F32, EAGLE_EINVAL);
  EAGLE_REQUIRE(hd == 64 || hd == 128, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(((uintptr_t)workspace & 255) == 0, EAGLE_EINVAL);
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_tree | (uintptr_t)v_tree | (uintptr_t)out |
                       (uintptr_t)k_cache | (uintptr_t)v_cache;
  EAGLE_REQUIRE((al & 15) == 0 && ((uintptr_t)mask & 7) == 0, EAGLE_EINVAL);
  const AttnPlan pl = attn_plan(Tq, Hq, Hkv, hd, L, in_dt);
  EAGLE_REQUIRE(pl.n_split + 1 <= kMergeSplits, EAGLE_EUNSUPPORTED);
  // 32-bit byte offsets within one slice
  EAGLE_REQUIRE(in_dt != EAGLE_BF16 || pl.tiles_per_split <= 65536, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(ws_bytes >= pl.total, EAGLE_EWORKSPACE);
  char* ws = (char*)workspace;
  AttnParams p{};
  p.q = (const bf16_t*)q;
  p.kc = (const bf16_t*)k_cache;
  p.vc = (const bf16_t*)v_cache;
  p.kt = (const bf16_t*)k_tree;
  p.vt = (const bf16_t*)v_tree;
  p.L = L;
  p.ldc = ld_cache;
  p.Tk = Tk;
  p.ldt = ld_tree;
  p.mask = mask;
  p.words = words;
  p.mask_rows = mask_rows;
  p.qmap = q_mask_row;
  p.Tq = Tq;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.c = scale * kLog2e;
  p.n_split = pl.n_split;
  p.tiles_per_split = pl.tiles_per_split;
  p.part_o = ws + pl.o_off;
  p.part_ml = (float2*)(ws + pl.ml_off);
  p.status = dev_status;
  if (in_dt == EAGLE_BF16) {
    const dim3 grid(pl.n_split + 1, Hkv, pl.qgroups);
    if (hd == 128) {
      if (pl.ntw == 1) launch_attn<128, 1, 4>(p, grid, stream);
      else if (pl.nw == 4) launch_attn<128, 2, 4>(p, grid, stream);
      else launch_ring<2, 8, 4>(p, grid, stream);
    } else {
      if (pl.ntw == 1) launch_attn<64, 1, 4>(p, grid, stream);
      else if (pl.nw == 4) launch_attn<64, 2, 4>(p, grid, stream);
      else launch_attn<64, 2, 8>(p, grid, stream);
    }
  } else {
    hipLaunchKernelGGL(tree_attn_f32_kernel, dim3(pl.n_split + 1, Tq * Hq), dim3(256), 0, stream,
                       p, hd);
  }
  EAGLE_LAUNCH_CHECK();
  const int RT = Tq * Hq;
  const int obf = out_dt == EAGLE_BF16 ? 1 : 0;
  if (in_dt == EAGLE_BF16) {
    if (hd == 128)
      hipLaunchKernelGGL(attn_merge_bf16_kernel<128>, dim3((RT + 3) / 4), dim3(256),
                         (size_t)4 * (pl.n_split + 1) * sizeof(float), stream,
                         (const bf16_t*)p.part_o, p.part_ml, pl.n_split + 1, RT, p.c, out, obf);
    else
      hipLaunchKernelGGL(attn_merge_bf16_kernel<64>, dim3((RT + 7) / 8), dim3(256),
                         (size_t)8 * (pl.n_split + 1) * sizeof(float), stream,
                         (const bf16_t*)p.part_o, p.part_ml, pl.n_split + 1, RT, p.c, out, obf);
  } else {
    hipLaunchKernelGGL(attn_merge_f32_kernel, dim3(RT), dim3(128), 0, stream,
                       (const float*)p.part_o, p.part_ml, pl.n_split + 1, RT, hd, p.c, out, obf);
  }

  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
