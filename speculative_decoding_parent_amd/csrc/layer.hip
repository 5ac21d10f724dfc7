// Decoder-layer support for the draft and verify passes of one cycle.
//
// Sources: "EAGLE-2: Feature-Level Speculative Decoding Guide", Key
// Architectural Mechanics 1 - the draft step h = W_fuse [f ; Emb(y)],
// f' = TransformerLayer(h); "Support Eagle-3 Speculative Decoding in llama.cpp"
// - the yuhuili/EAGLE3-LLaMA3.1-Instruct-8B printout (q/k/v/o projections, a
// SiLU-gated MLP 4096 -> 14336 -> 4096, RMSNorms with eps 1e-5, rotary
// embedding, no biases) and the draft sharing the target's embedding.
//
// Projections use the weight-streaming MFMA core (few rows, every weight byte
// read once from HBM) with two epilogues: plain (+ an fp32 residual) and SwiGLU
// (each wave streams 32 gate rows and the 32 matching up rows, so silu(g) * u is
// formed in registers and only the product is written).  The residual stream
// stays fp32; only MFMA operands (normed activations, attention output, MLP
// hidden) are bf16.  RoPE angles are formed and rotated in fp64 (positions up
// to ~37K make fp32 angles lose ~1e-3 rad).
#include <algorithm>

#include "wstream.h"

namespace eagle {


struct LinParams {
  const bf16_t* x;
  int M, K;
  const bf16_t* w0;   // plain: W [N][K]; swiglu: W_gate [N][K]
  const bf16_t* w1;   // swiglu: W_up [N][K]
  int N;
  const float* residual;   // plain, nullable: [M][N]
  void* out;               // [M][N]
  int out_bf16;
  int ksplit;              // k slices (blockIdx.y)
  float* part;             // [ksplit][1 or 2][M][N]
  int to_part;             // write fp32 partials for a separate epilogue kernel
  RowNorm in;              // deferred RMSNorm of the input rows (in.ssq null: none)
};

__device__ __forceinline__ void store4(void* out, int out_bf16, size_t off, int n, int N,
                                       const float (&y)[4]) {
  if (out_bf16) {
    bf16_t* o = (bf16_t*)out + off;
    if ((N & 3) == 0 && n + 3 < N) {
      *(u32x2*)o = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < N) o[j] = (bf16_t)f32_to_bf16_bits(y[j]);
    }
  } else {
    float* o = (float*)out + off;
    if ((N & 3) == 0 && n + 3 < N) {
      *(f32x4*)o = f32x4{y[0], y[1], y[2], y[3]};
    } else {
      for (int j = 0; j < 4; ++j)
        if (n + j < N) o[j] = y[j];
    }
  }
}

// W tiles (16 rows) per wave: fewer as more activation rows need accumulators
// (no register spills up to M = 256).  A SwiGLU wave pairs MT/2 gate tiles
// with the MT/2 up tiles of the same output columns.
__host__ __device__ constexpr int lin_mt(int nt, int swiglu) {
  return nt <= 2 ? 4 : (nt <= 8 || swiglu ? 2 : 1);
}
__host__ __device__ constexpr int lin_cols_block(int mt, int swiglu) {
  return swiglu ? 4 * 8 * mt : 4 * 16 * mt;
}

// RR: W read in 256-byte row runs through a wave-private LDS tile (the
// streaming core's row-run variant) instead of 16-row operand-layout loads;
// chosen by the host for long k ranges, where it streams faster.
template <int NT, int SWIGLU, int MT, bool RR>
__global__ __launch_bounds__(256, (NT * MT <= 8 ? 2 : 1)) void linear_bf16_kernel(LinParams p) {
  static_assert(!SWIGLU || MT % 2 == 0, "SwiGLU pairs gate and up tiles");
  constexpr int HALF = SWIGLU ? MT / 2 : MT;      // output tiles per wave
  __shared__ __attribute__((aligned(16))) bf16_t fs[ws_lds_elems<NT>()];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int n0 = blockIdx.x * lin_cols_block(MT, SWIGLU) + wave * 16 * HALF;
  const bf16_t* wrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int col = n0 + (mt % HALF) * 16 + r16;
    const bf16_t* w = (SWIGLU && mt >= HALF) ? p.w1 : p.w0;
    wrow[mt] = w + (size_t)min(col, p.N - 1) * p.K + g * 8;
  }
  // k slice of this workgroup
  const int kc = p.K / p.ksplit;
  const int k0 = blockIdx.y * kc;
  f32x4 acc[MT][NT];
  __shared__ __attribute__((aligned(16))) char wlds[RR ? 4 : 1][RR ? MT * 4096 : 16];
  if constexpr (RR) {
    int trow[MT], wsel[MT];
    const int n0s = __builtin_amdgcn_readfirstlane(n0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      trow[mt] = n0s + (mt % HALF) * 16;
      wsel[mt] = (SWIGLU && mt >= HALF) ? 1 : 0;
    }
    wstream_mfma_rr<NT, MT, false>(p.w0 + k0, SWIGLU ? p.w1 + k0 : nullptr, p.N, p.K, trow, wsel,
                                   p.x + k0, p.K, p.M, kc, fs, wlds[wave], acc);
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) wrow[mt] += k0;
    wstream_mfma<NT, MT>(wrow, p.x + k0, p.K, p.M, kc, fs, acc);
  }

  if (p.to_part) {
    // fp32 partials; a SwiGLU wave's up tiles go to plane 1
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int m = nt * 16 + r16;
      if (m >= p.M) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int n = n0 + (mt % HALF) * 16 + 4 * g;
        if (n >= p.N) continue;
        const int plane = mt / HALF;
        const size_t off =
            (((size_t)blockIdx.y * (SWIGLU ? 2 : 1) + plane) * p.M + m) * p.N + n;
        const float y[4] = {acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]};
        store4(p.part, 0, off, n, p.N, y);
      }
    }
    return;
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int m = nt * 16 + r16;
    if (m >= p.M) continue;
    const float rs = p.in.ssq ? row_norm_scale(p.in, p.M, m) : 1.0f;
#pragma unroll
    for (int mt = 0; mt < HALF; ++mt) {
      const int n = n0 + mt * 16 + 4 * g;
      if (n >= p.N) continue;
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (SWIGLU) {
          const float gt = acc[mt][nt][j] * rs;
          y[j] = gt / (1.0f + expf(-gt)) * (acc[mt + HALF][nt][j] * rs);
        } else {
          y[j] = acc[mt][nt][j] * rs;
          if (p.residual && n + j < p.N) y[j] += p.residual[(size_t)m * p.N + n + j];
        }
      }
      store4(p.out, SWIGLU ? 1 : p.out_bf16, (size_t)m * p.N + n, n, p.N, y);
    }
  }
}

// Sum the k-slice partials in slice order and apply the epilogue: plain
// (+ residual) or SwiGLU (silu(sum gate) * sum up).  4 outputs per thread,
// 16-byte loads when N % 4 == 0.
__global__ __launch_bounds__(256) void linear_reduce_kernel(LinParams p, int swiglu) {
  const size_t MN = (size_t)p.M * p.N;
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= MN) return;
  const int planes = swiglu ? 2 : 1;
  const size_t stride = (size_t)planes * MN;
  float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
  const bool vec = (p.N & 3) == 0;
  if (vec) {
    f32x4 va = {0.f, 0.f, 0.f, 0.f}, vb = {0.f, 0.f, 0.f, 0.f};
    const float* pa = p.part + e0;
#pragma unroll 8
    for (int s = 0; s < p.ksplit; ++s) {
      va += *(const f32x4*)(pa + s * stride);
      if (swiglu) vb += *(const f32x4*)(pa + s * stride + MN);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = va[j];
      b[j] = vb[j];
    }
  } else {
    for (int s = 0; s < p.ksplit; ++s) {
      const float* pa = p.part + (size_t)s * stride;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (e0 + j >= MN) break;
        a[j] += pa[e0 + j];
        if (swiglu) b[j] += pa[MN + e0 + j];
      }
    }
  }
  if (p.in.ssq) {
    if (vec) {   // the four outputs share a row
      const float rs = row_norm_scale(p.in, p.M, (int)(e0 / p.N));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] *= rs;
        b[j] *= rs;
      }
    } else {
      for (int j = 0; j < 4; ++j) {
        if (e0 + j >= MN) break;
        const float rs = row_norm_scale(p.in, p.M, (int)((e0 + j) / p.N));
        a[j] *= rs;
        b[j] *= rs;
      }
    }
  }
  float y[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (swiglu) {
      y[j] = a[j] / (1.0f + expf(-a[j])) * b[j];
    } else {
      y[j] = a[j];
      if (p.residual && e0 + j < MN) y[j] += p.residual[e0 + j];
    }
  }
  const int m = (int)(e0 / p.N);
  const int n = (int)(e0 - (size_t)m * p.N);
  if (vec) {
    store4(p.out, swiglu ? 1 : p.out_bf16, e0, n, p.N, y);
  } else {
    for (int j = 0; j < 4 && e0 + j < MN; ++j) {
      if (swiglu || p.out_bf16)
        ((bf16_t*)p.out)[e0 + j] = (bf16_t)f32_to_bf16_bits(y[j]);
      else
        ((float*)p.out)[e0 + j] = y[j];
    }
  }
}

// Row-wise reduce epilogues: one workgroup per row m sums the row's k-slice
// partials (slice order) so the whole row is available to a row operation.
constexpr int kRowThreads = 512;
constexpr int kRowVec = 4;                    // float4 per thread: N <= 8192
constexpr int kRowMaxN = kRowThreads * 4 * kRowVec;

__device__ __forceinline__ f32x4 sum_slices4(const LinParams& p, size_t off) {
  const size_t MN = (size_t)p.M * p.N;
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < p.ksplit; ++s) a += *(const f32x4*)(p.part + s * MN + off);
  return a;
}

// out = sum + residual (fp32), then norm_out = RMSNorm(out) * gamma (bf16):
// one workgroup per row m.
__global__ __launch_bounds__(kRowThreads) void linear_reduce_norm_kernel(
    LinParams p, const float* __restrict__ gamma, float eps, bf16_t* __restrict__ norm_out) {
  __shared__ float red[kRowThreads / 64];
  const int m = blockIdx.x;
  const int N = p.N;
  f32x4 v[kRowVec];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kRowVec; ++q) {
    const int n = (threadIdx.x + kRowThreads * q) * 4;
    v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (n >= N) continue;
    const size_t off = (size_t)m * N + n;
    v[q] = sum_slices4(p, off);
    if (p.residual) v[q] += *(const f32x4*)(p.residual + off);
    *(f32x4*)((float*)p.out + off) = v[q];
#pragma unroll
    for (int j = 0; j < 4; ++j) ss = fmaf(v[q][j], v[q][j], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kRowThreads / 64; ++w) tot += red[w];
  const float r = 1.0f / sqrtf(tot / (float)N + eps);
#pragma unroll
  for (int q = 0; q < kRowVec; ++q) {
    const int n = (threadIdx.x + kRowThreads * q) * 4;
    if (n >= N) continue;
    const f32x4 gm = *(const f32x4*)(gamma + n);
    *(u32x2*)(norm_out + (size_t)m * N + n) =
        u32x2{pack_bf16x2(v[q][0] * r * gm[0], v[q][1] * r * gm[1]),
              pack_bf16x2(v[q][2] * r * gm[2], v[q][3] * r * gm[3])};
  }
}

// The deferred form over column chunks: workgroup (m, c) sums the k-slice
// partials of row m's columns [c kRedCols, (c + 1) kRedCols) (slice order),
// adds the residual, writes out (fp32) and xg = out * gamma (bf16), and the
// chunk's sum of squares to ssq_out[c][m]: one part per chunk, so a whole
// row needs no single workgroup.
constexpr int kRedCols = 1024;
__global__ __launch_bounds__(256) void linear_reduce_dnorm_kernel(LinParams p,
                                                                  const float* __restrict__ gamma,
                                                                  bf16_t* __restrict__ xg_out,
                                                                  float* __restrict__ ssq_out) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int c = blockIdx.y;
  const int N = p.N;
  const int n = c * kRedCols + threadIdx.x * 4;
  float ss = 0.f;
  if (n < N) {
    const size_t off = (size_t)m * N + n;
    f32x4 v = sum_slices4(p, off);
    if (p.residual) v += *(const f32x4*)(p.residual + off);
    *(f32x4*)((float*)p.out + off) = v;
#pragma unroll
    for (int j = 0; j < 4; ++j) ss = fmaf(v[j], v[j], ss);
    const f32x4 gm = *(const f32x4*)(gamma + n);
    *(u32x2*)(xg_out + off) = u32x2{pack_bf16x2(v[0] * gm[0], v[1] * gm[1]),
                                    pack_bf16x2(v[2] * gm[2], v[3] * gm[3])};
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) ssq_out[(size_t)c * p.M + m] = ((red[0] + red[1]) + red[2]) + red[3];
}

// cos and sin of the rotary angle pos * inv: the angle is formed and reduced
// to [-pi, pi] in fp64 (positions reach ~37K, where an fp32 angle would be off
// by ~1e-3 rad), sin and cos are then taken in fp32 (~1e-7 absolute).
__device__ __forceinline__ void rope_cs(double pos, double inv, float& c, float& s) {
  const double a = pos * inv;
  const double red = a - 6.283185307179586 * rint(a * 0.15915494309189535);
  sincosf((float)red, &s, &c);
}

struct RopeArgs {
  int Hq, Hkv, hd;
  const int32_t* depth;
  int64_t pos_base;
  double theta;
  const int32_t* row_slot;
  int slot_cap;
  bf16_t* q_out;
  bf16_t* k_tree;
  bf16_t* v_tree;
  int ld_tree;
  int32_t* status;
};

// Rotate heads [h0, h1) of one row held in LDS (row[] starts at head h0; q
// heads, then k heads, then v heads of hd) and place them: q -> q_out[m],
// rotated k and plain v -> tree slot row_slot[m].
__device__ void rope_place_row(const float* row, int m, const RopeArgs& r, const double* inv,
                               int h0, int h1) {
  const int half = r.hd / 2;
  int slot = r.row_slot ? r.row_slot[m] : m;
  if (slot < 0 || slot >= r.slot_cap) {
    if (threadIdx.x == 0) set_status(r.status, EAGLE_DEV_BAD_INDEX);
    slot = -1;
  }
  const double pos = (double)(r.pos_base + r.depth[m]);
  for (int e = threadIdx.x; e < (h1 - h0) * half; e += blockDim.x) {
    const int hl = e / half;
    const int hh = h0 + hl;
    const int i = e - hl * half;
    const float x1 = row[hl * r.hd + i];
    const float x2 = row[hl * r.hd + i + half];
    if (hh < r.Hq + r.Hkv) {
      float cs, sn;
      rope_cs(pos, inv[i], cs, sn);
      const float y1 = x1 * cs - x2 * sn;
      const float y2 = x2 * cs + x1 * sn;
      if (hh < r.Hq) {
        bf16_t* q = r.q_out + ((size_t)m * r.Hq + hh) * r.hd;
        q[i] = (bf16_t)f32_to_bf16_bits(y1);
        q[i + half] = (bf16_t)f32_to_bf16_bits(y2);
      } else if (slot >= 0) {
        bf16_t* k = r.k_tree + ((size_t)(hh - r.Hq) * r.ld_tree + slot) * r.hd;
        k[i] = (bf16_t)f32_to_bf16_bits(y1);
        k[i + half] = (bf16_t)f32_to_bf16_bits(y2);
      }
    } else if (slot >= 0) {
      bf16_t* v = r.v_tree + ((size_t)(hh - r.Hq - r.Hkv) * r.ld_tree + slot) * r.hd;
      v[i] = (bf16_t)f32_to_bf16_bits(x1);
      v[i + half] = (bf16_t)f32_to_bf16_bits(x2);
    }
  }
}

constexpr int kRopeMaxHalf = 128;

// qkv projection epilogue: workgroup (m, group) sums the partials of row m's
// heads [kRopeHeads group, ...) into LDS, then RoPE + place.
constexpr int kRopeHeads = 8;
__global__ __launch_bounds__(256) void linear_reduce_rope_kernel(LinParams p, RopeArgs r) {
  extern __shared__ float row[];
  __shared__ double inv[kRopeMaxHalf];
  const int m = blockIdx.x;
  const int H = r.Hq + 2 * r.Hkv;
  const int h0 = blockIdx.y * kRopeHeads;
  const int h1 = min(H, h0 + kRopeHeads);
  const int half = r.hd / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x)
    inv[i] = pow(r.theta, -2.0 * (double)i / (double)r.hd);
  const float rs = p.in.ssq ? row_norm_scale(p.in, p.M, m) : 1.0f;
  const int c0 = h0 * r.hd, nc = (h1 - h0) * r.hd;
  for (int n = threadIdx.x * 4; n < nc; n += 256 * 4)
    *(f32x4*)(row + n) = sum_slices4(p, (size_t)m * p.N + c0 + n) * rs;
  __syncthreads();
  rope_place_row(row, m, r, inv, h0, h1);
}

// out[m] = x[m] / sqrt(mean(x[m]^2) + eps) * gamma, fp32 in, bf16 out.  One
// workgroup per row; rows of up to 256 * 4 * kNormVec elements stay in
// registers between the sum of squares and the scaling (one pass over HBM).
constexpr int kNormVec = 8;

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x,
                                                      const float* __restrict__ gamma, int N,
                                                      float eps, bf16_t* __restrict__ out) {
  __shared__ float red[4];
  const float* row = x + (size_t)blockIdx.x * N;
  bf16_t* o = out + (size_t)blockIdx.x * N;
  const bool inreg = (N & 3) == 0 && N <= 256 * 4 * kNormVec &&
                     (((uintptr_t)x | (uintptr_t)gamma | (uintptr_t)out) & 15) == 0;
  f32x4 v[kNormVec];
  float ss = 0.f;
  if (inreg) {
#pragma unroll
    for (int q = 0; q < kNormVec; ++q) {
      const int n = (threadIdx.x + 256 * q) * 4;
      v[q] = n < N ? *(const f32x4*)(row + n) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = fmaf(v[q][j], v[q][j], ss);
    }
  } else {
    for (int n = threadIdx.x; n < N; n += 256) ss = fmaf(row[n], row[n], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float r = 1.0f / sqrtf(tot / (float)N + eps);
  if (inreg) {
#pragma unroll
    for (int q = 0; q < kNormVec; ++q) {
      const int n = (threadIdx.x + 256 * q) * 4;
      if (n >= N) continue;
      const f32x4 gm = *(const f32x4*)(gamma + n);
      *(u32x2*)(o + n) = u32x2{pack_bf16x2(v[q][0] * r * gm[0], v[q][1] * r * gm[1]),
                               pack_bf16x2(v[q][2] * r * gm[2], v[q][3] * r * gm[3])};
    }
  } else {
    for (int n = threadIdx.x; n < N; n += 256)
      o[n] = (bf16_t)f32_to_bf16_bits(row[n] * r * gamma[n]);
  }
}

// qkv [M][(Hq + 2 Hkv) hd] fp32 -> q_out [M][Hq][hd] bf16 (rotated); k (rotated)
// and v into the tree K/V at slot row_slot[m].  Rotation pairs dims i and
// i + hd/2 by angle (pos_base + depth[m]) * theta^(-2i/hd).
__global__ __launch_bounds__(256) void rope_qkv_kernel(const float* __restrict__ qkv, RopeArgs r) {
  __shared__ double inv[kRopeMaxHalf];
  const int m = blockIdx.x;
  const int half = r.hd / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x)
    inv[i] = pow(r.theta, -2.0 * (double)i / (double)r.hd);
  __syncthreads();
  rope_place_row(qkv + (size_t)m * (r.Hq + 2 * r.Hkv) * r.hd, m, r, inv, 0, r.Hq + 2 * r.Hkv);
}

// One draft round's preparation, one workgroup per row j (frontier entry f):
// bookkeeping (slot base + j, the parent's slot, token, depth), the slot's
// ancestor mask row (its parent slot's row plus its own bit) and the fused
// input row [bf16(feature of the parent slot, or the root feature) ; Emb(token)].
// Parents belong to earlier rounds, so no row reads what another row writes.
__global__ __launch_bounds__(256) void draft_prepare_kernel(
    const int32_t* __restrict__ frontier, const int32_t* __restrict__ pool_token,
    const int32_t* __restrict__ pool_parent, const int32_t* __restrict__ pool_depth, int pool_n,
    int32_t* __restrict__ slot_of_pool, int slot_base, int slot_cap,
    int32_t* __restrict__ slot_parent, uint64_t* __restrict__ slot_mask, int words,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_depth,
    int32_t* __restrict__ row_slot, int32_t* __restrict__ row_src, const float* __restrict__ feat,
    const float* __restrict__ root_feat, const bf16_t* __restrict__ embed, int V, int d,
    bf16_t* __restrict__ x_in, int32_t* __restrict__ status) {
  __shared__ int sh_src, sh_tok;
  const int j = blockIdx.x;
  const int slot = slot_base + j;
  if (threadIdx.x == 0) {
    int f = frontier[j];
    if (f < 0 || f >= pool_n) {
      set_status(status, EAGLE_DEV_BAD_INDEX);
      f = 0;
    }
    const int par = pool_parent[f];
    int src = -1;
    if (par >= 0) {
      src = par < pool_n ? slot_of_pool[par] : -1;
      if (src < 0 || src >= slot_base) {
        set_status(status, EAGLE_DEV_BAD_INDEX);
        src = -1;
      }
    }
    int tok = pool_token[f];
    if (tok < 0 || tok >= V) {
      set_status(status, EAGLE_DEV_BAD_TOKEN);
      tok = 0;
    }
    slot_of_pool[f] = slot;
    slot_parent[slot] = src;
    row_token[j] = tok;
    row_depth[j] = pool_depth[f];
    row_slot[j] = slot;
    row_src[j] = src;
    sh_src = src;
    sh_tok = tok;
  }
  __syncthreads();
  const int src = sh_src;
  if (slot_mask && (int)threadIdx.x < words) {
    const int w = threadIdx.x;
    uint64_t m = src >= 0 ? slot_mask[(size_t)src * words + w] : 0ull;
    if ((slot >> 6) == w) m |= 1ull << (slot & 63);
    slot_mask[(size_t)slot * words + w] = m;
  }
  if (x_in) {
    const float* f = src >= 0 ? feat + (size_t)src * d : root_feat;
    const bf16_t* e = embed + (size_t)sh_tok * d;
    bf16_t* o = x_in + (size_t)j * 2 * d;
    if ((d & 7) == 0 && (((uintptr_t)f | (uintptr_t)e | (uintptr_t)o) & 15) == 0) {
      for (int n = threadIdx.x * 8; n < d; n += 256 * 8) {
        const f32x4 a = *(const f32x4*)(f + n);
        const f32x4 b = *(const f32x4*)(f + n + 4);
        *(u32x4*)(o + n) = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                 pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
        *(u32x4*)(o + d + n) = *(const u32x4*)(e + n);
      }
    } else {
      for (int n = threadIdx.x; n < d; n += 256) {
        o[n] = (bf16_t)f32_to_bf16_bits(f[n]);
        o[d + n] = e[n];
      }
    }
  }
}

// out[m] = float(embed[token[m]])
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ token,
                                                    const bf16_t* __restrict__ embed, int V, int d,
                                                    float* __restrict__ out,
                                                    int32_t* __restrict__ status) {
  const int m = blockIdx.x;
  int tok = token[m];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0) set_status(status, EAGLE_DEV_BAD_TOKEN);
    tok = 0;
  }
  const bf16_t* e = embed + (size_t)tok * d;
  float* o = out + (size_t)m * d;
  if ((d & 7) == 0 && (((uintptr_t)e | (uintptr_t)o) & 15) == 0) {
    for (int n = threadIdx.x * 8; n < d; n += 256 * 8) {
      const u32x4 b = *(const u32x4*)(e + n);
      *(f32x4*)(o + n) = f32x4{bf16_bits_to_f32(b[0] & 0xffffu), bf16_bits_to_f32(b[0] >> 16),
                               bf16_bits_to_f32(b[1] & 0xffffu), bf16_bits_to_f32(b[1] >> 16)};
      *(f32x4*)(o + n + 4) = f32x4{bf16_bits_to_f32(b[2] & 0xffffu), bf16_bits_to_f32(b[2] >> 16),
                                   bf16_bits_to_f32(b[3] & 0xffffu), bf16_bits_to_f32(b[3] >> 16)};
    }
  } else {
    for (int n = threadIdx.x; n < d; n += 256) o[n] = bf16_bits_to_f32(e[n]);
  }
}

// out[m] = float(embed[token[m]]) with the norm that follows deferred:
// xg[m] = bf16(out[m] * gamma) and ssq[m] = sum_n out[m][n]^2 (one part).
__global__ __launch_bounds__(256) void embed_deferred_kernel(
    const int32_t* __restrict__ token, const bf16_t* __restrict__ embed, int V, int d,
    const float* __restrict__ gamma, float* __restrict__ out, bf16_t* __restrict__ xg,
    float* __restrict__ ssq, int32_t* __restrict__ status) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  int tok = token[m];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0) set_status(status, EAGLE_DEV_BAD_TOKEN);
    tok = 0;
  }
  const bf16_t* e = embed + (size_t)tok * d;
  float* o = out + (size_t)m * d;
  bf16_t* x = xg + (size_t)m * d;
  float ss = 0.f;
  for (int n = threadIdx.x * 8; n < d; n += 256 * 8) {   // d % 8 == 0
    const u32x4 b = *(const u32x4*)(e + n);
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32(b[j] & 0xffffu);
      v[2 * j + 1] = bf16_bits_to_f32(b[j] >> 16);
    }
    *(f32x4*)(o + n) = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)(o + n + 4) = f32x4{v[4], v[5], v[6], v[7]};
    const f32x4 g0 = *(const f32x4*)(gamma + n);
    const f32x4 g1 = *(const f32x4*)(gamma + n + 4);
    *(u32x4*)(x + n) = u32x4{pack_bf16x2(v[0] * g0[0], v[1] * g0[1]),
                             pack_bf16x2(v[2] * g0[2], v[3] * g0[3]),
                             pack_bf16x2(v[4] * g1[0], v[5] * g1[1]),
                             pack_bf16x2(v[6] * g1[2], v[7] * g1[3])};
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) ssq[m] = ((red[0] + red[1]) + red[2]) + red[3];
}

// ---------------------------------------------------------------- few rows
//
// Projections of M <= 16 activation rows (the draft rounds) run as ONE kernel
// each, epilogue included.  A workgroup owns 64 weight rows (4 MFMA tiles of
// 16) and a range of 128-wide k steps; its four waves take interleaved steps of
// that range, each streaming W from HBM in 256-byte row runs (non-temporal)
// through a wave-private LDS tile into MFMA A operands, and the activation
// rows straight from L2 into B operands (no barrier in the loop); the four
// wave tiles are added in LDS.  A column
// block's k range is split over S workgroups so that ~256 are in flight; each
// writes its fp32 tile to the workspace and the last one to arrive (a
// per-column-block counter) sums the S tiles in range order, so the result
// does not depend on scheduling, and runs the epilogue:
//   plain   out = y (+ residual), fp32 or bf16
//   ressq   out = y + residual (fp32), xg = out * gamma (bf16) and the row sums
//           of squares of its 64 columns: a deferred RMSNorm (RowNorm) whose
//           row scale the next product applies
//   rope    the workgroup owns columns i and i + hd/2 of one head, so q and k
//           are rotated in registers and q, k, v are placed directly
//   swiglu  the workgroup owns 32 gate rows and the 32 matching up rows
// Inputs may carry a deferred RMSNorm (p.in): its row scale multiplies the
// summed tile before the epilogue.  Counters live in the first
// kSkCounterBytes of the workspace: they must be zero before the first call,
// and every call leaves them zero.
constexpr int kSkMT = 4;
constexpr size_t kSkCounterBytes = 64 * 1024;
constexpr int kSkMaxBlocks = (int)(kSkCounterBytes / 4);
constexpr int kSkMaxRows = 16;
constexpr int kSkMaxS = 16;     // k ranges per column block

enum SkMode { SK_PLAIN = 0, SK_RESSQ = 1, SK_ROPE = 2, SK_SWIGLU = 3 };

struct SkParams {
  const bf16_t* x;
  int M, K;
  const bf16_t* w0;        // W, or W_gate
  const bf16_t* w1;        // W_up
  int N;                   // output columns (rope: (Hq + 2 Hkv) hd)
  int nblk, S;
  const float* residual;
  void* out;
  int out_bf16;
  const float* gamma;      // ressq
  bf16_t* xg_out;          // ressq: [M][N]
  float* ssq_out;          // ressq: [nblk][M]
  int32_t* ctr;            // [nblk] per column block
  float* part;             // [S][nblk][M][64]
  int nsub;                // rope: column blocks per head
  RopeArgs rope;
  RowNorm in;
  const bf16_t* xseg[3];   // kseg > 0: x is these three [M][kseg] blocks side by side
  int kseg;
};

// First weight row of tile mt (0..3) of column block xb.
template <int MODE>
__device__ __forceinline__ int sk_wrow(const SkParams& p, int xb, int mt) {
  if (MODE == SK_SWIGLU) return xb * 32 + (mt & 1) * 16;
  if (MODE == SK_ROPE) {
    const int hd = p.rope.hd;
    const int h = xb / p.nsub, sub = xb - h * p.nsub;
    return h * hd + (mt >= 2 ? hd / 2 : 0) + sub * 32 + (mt & 1) * 16;
  }
  return xb * 64 + mt * 16;
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void linear_rows_kernel(SkParams p) {
  // a wave's k step of W (row runs, see below); after the loop each wave's
  // first 4 KB hold its tiles for the sum over the waves
  __shared__ __attribute__((aligned(16))) char wlds[4][kSkMT * 4096];
  __shared__ float ssl[4][kSkMaxRows];
  __shared__ float rsc[kSkMaxRows];
  __shared__ double sinv[MODE == SK_ROPE ? kRopeMaxHalf : 1];
  __shared__ int flag;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  const int xb = blockIdx.x;
  const int yb = blockIdx.y;
  const int M = p.M, K = p.K, N = p.N;
  if (MODE == SK_ROPE && threadIdx.x < p.rope.hd / 2)   // read after the first barrier
    sinv[threadIdx.x] = pow(p.rope.theta, -2.0 * (double)threadIdx.x / (double)p.rope.hd);
  // input row scales: lanes (row rm, q0) add the partials q0, q0 + 16, ... of
  // row rm; the loads overlap the main loop, the sums are finished after it
  const int rm = threadIdx.x >> 4, q0 = threadIdx.x & 15;
  const bool has_in = p.in.ssq && rm < M;
  float in_part[kPartBatch];
  if (has_in) strided_load(p.in.ssq + rm, p.in.parts, (size_t)M, q0, 16, in_part);

  // W is read in runs of 256 bytes per row with non-temporal loads (load
  // instruction i of tile mt: lane l takes row 4 i + l / 16 of the tile, bytes
  // 16 (l % 16) of the k step) and passed through the wave's LDS tile into the
  // MFMA operand layout.  Buffer ranges start at the workgroup's first row of
  // each matrix (rows past N read zero).
  const int wrow0 = sk_wrow<MODE>(p, xb, 0);
  const int wspan = MODE == SK_ROPE ? p.rope.hd : 64;
  const int wrows = max(0, min(wspan, N - wrow0));
  const size_t wbytes = (size_t)wrows * K * sizeof(bf16_t);
  const __amdgpu_buffer_rsrc_t wrs0 = buf_rsrc(p.w0 + (size_t)wrow0 * K, wbytes);
  const __amdgpu_buffer_rsrc_t wrs1 =
      buf_rsrc((MODE == SK_SWIGLU ? p.w1 : p.w0) + (size_t)wrow0 * K, wbytes);
  uint32_t wvo[kSkMT];
#pragma unroll
  for (int mt = 0; mt < kSkMT; ++mt)
    wvo[mt] = (uint32_t)((sk_wrow<MODE>(p, xb, mt) - wrow0 + g) * K * sizeof(bf16_t)) + r16 * 16;
  const uint32_t wistride = 4u * K * sizeof(bf16_t);
  char* wl = wlds[wave];
  const bool xok = r16 < M;
  const int xrow = min(r16, M - 1);
  const bf16_t* xr = p.x + (size_t)xrow * K + g * 8;
  const int nk = K / kWsKG;
  const int kb = (int)((int64_t)yb * nk / p.S);
  const int ke = (int)((int64_t)(yb + 1) * nk / p.S);

  f32x4 acc[kSkMT];
#pragma unroll
  for (int mt = 0; mt < kSkMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 wa[kSkMT][4], wb[kSkMT][4], xa[4], xbv[4];
  auto load = [&](int kk, u32x4 (&w)[kSkMT][4], u32x4 (&xv)[4]) {
    const bf16_t* xp = xr + kk * kWsKG;
    if (p.kseg) {  // a 128-wide k step lies inside one segment (kseg % 128 == 0)
      const int kel = kk * kWsKG;
      const int sg = kel / p.kseg;
      xp = p.xseg[sg] + (size_t)xrow * p.kseg + (kel - sg * p.kseg) + g * 8;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xv[i] = xok ? *(const u32x4*)(xp + i * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int mt = 0; mt < kSkMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[mt][i] = __builtin_amdgcn_raw_buffer_load_b128(
            (MODE == SK_SWIGLU && mt >= 2) ? wrs1 : wrs0, wvo[mt],
            (uint32_t)(i * wistride + kk * kWsKG * sizeof(bf16_t)), kNtPolicy);
  };
  auto compute = [&](const u32x4 (&w)[kSkMT][4], const u32x4 (&xv)[4]) {
    // to the operand layout: row r of a tile at r * 256, 16-byte chunk c at
    // (c ^ r) * 16 (64 distinct banks per 16 lanes, writes and reads alike)
#pragma unroll
    for (int mt = 0; mt < kSkMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + g;
        *(u32x4*)(wl + mt * 4096 + row * 256 + ((r16 ^ row) << 4)) = w[mt][i];
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 b = ws_as_bf16x8(xv[i]);
#pragma unroll
      for (int mt = 0; mt < kSkMT; ++mt) {
        const bf16x8 a = *(const bf16x8*)(wl + mt * 4096 + r16 * 256 + (((4 * i + g) ^ r16) << 4));
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
      }
    }
  };
  int kk = kb + wave;
  if (kk < ke) load(kk, wa, xa);
  for (; kk < ke; kk += 8) {
    if (kk + 4 < ke) load(kk + 4, wb, xbv);
    compute(wa, xa);
    if (kk + 4 >= ke) break;
    if (kk + 8 < ke) load(kk + 8, wa, xa);
    compute(wb, xbv);
  }
  float in_ss = has_in ? strided_finish(p.in.ssq + rm, p.in.parts, (size_t)M, q0, 16, in_part) : 0.f;
  in_ss += dpp_move<kDppQuadXor1>(in_ss);      // the 16 lanes of a row: a DPP row
  in_ss += dpp_move<kDppQuadXor2>(in_ss);
  in_ss += dpp_move<kDppHalfMirror>(in_ss);
  in_ss += dpp_move<kDppRowMirror>(in_ss);
  if (q0 == 0 && rm < M)
    rsc[rm] = p.in.ssq ? 1.0f / sqrtf(in_ss / (float)p.in.n + p.in.eps) : 1.0f;
  // each wave's tiles go to the start of its own LDS tile (no other wave reads
  // that tile), then every wave reads all four
  auto redp = [&](int w, int mt) -> f32x4* {
    return (f32x4*)(wlds[w]) + mt * 64;
  };
#pragma unroll
  for (int mt = 0; mt < kSkMT; ++mt) redp(wave, mt)[lane] = acc[mt];
  __syncthreads();

  // tiles finished by this wave: one (plain, ressq) or a (first, second) pair
  constexpr bool kPair = MODE == SK_ROPE || MODE == SK_SWIGLU;
  const bool owner = kPair ? wave < 2 : true;
  const int ta = wave, tb = wave + 2;
  const int m = r16;
  f32x4 ya = redp(0, ta & 3)[lane] + redp(1, ta & 3)[lane];
  ya = ya + redp(2, ta & 3)[lane];
  ya = ya + redp(3, ta & 3)[lane];
  f32x4 yb2 = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kPair) {
    yb2 = redp(0, tb & 3)[lane] + redp(1, tb & 3)[lane];
    yb2 = yb2 + redp(2, tb & 3)[lane];
    yb2 = yb2 + redp(3, tb & 3)[lane];
  }
  if (p.S > 1) {
    const __amdgpu_buffer_rsrc_t rpart =
        dev_rsrc(p.part, (size_t)p.S * p.nblk * M * 64 * sizeof(float));
    // partial tile [yb][xb][m][64] (byte offsets)
    const uint32_t mine = (uint32_t)((((size_t)yb * p.nblk + xb) * M + m) * 64 * sizeof(float));
    if (owner && m < M) {
      st_dev4(rpart, mine + (ta * 16 + 4 * g) * 4, ya);
      if (kPair) st_dev4(rpart, mine + (tb * 16 + 4 * g) * 4, yb2);
    }
    if (!arrive_last(p.ctr + xb, p.S, &flag)) return;
    if (owner && m < M) {
      // all S tiles in flight at once, then summed in range order
      f32x4 ta4[kSkMaxS], tb4[kSkMaxS];
#pragma unroll
      for (int s = 0; s < kSkMaxS; ++s) {
        if (s < p.S) {
          const uint32_t o = (uint32_t)((((size_t)s * p.nblk + xb) * M + m) * 64 * sizeof(float));
          ta4[s] = ld_dev4(rpart, o + (ta * 16 + 4 * g) * 4);
          if (kPair) tb4[s] = ld_dev4(rpart, o + (tb * 16 + 4 * g) * 4);
        }
      }
      ya = f32x4{0.f, 0.f, 0.f, 0.f};
      yb2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kSkMaxS; ++s) {
        if (s < p.S) {
          ya = ya + ta4[s];
          if (kPair) yb2 = yb2 + tb4[s];
        }
      }
    }
  }
  if (m < M) {
    const float rs = rsc[m];
    ya = ya * rs;
    yb2 = yb2 * rs;
  }

  if (MODE == SK_PLAIN || MODE == SK_RESSQ) {
    const int n = xb * 64 + ta * 16 + 4 * g;
    float ss = 0.f;
    if (m < M && n < N) {
      float y[4] = {ya[0], ya[1], ya[2], ya[3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (p.residual && n + j < N) y[j] += p.residual[(size_t)m * N + n + j];
        if (n + j < N) ss = fmaf(y[j], y[j], ss);
      }
      store4(p.out, MODE == SK_RESSQ ? 0 : p.out_bf16, (size_t)m * N + n, n, N, y);
      if (MODE == SK_RESSQ) {   // N % 4 == 0
        const f32x4 gm = *(const f32x4*)(p.gamma + n);
        *(u32x2*)(p.xg_out + (size_t)m * N + n) =
            u32x2{pack_bf16x2(y[0] * gm[0], y[1] * gm[1]), pack_bf16x2(y[2] * gm[2], y[3] * gm[3])};
      }
    }
    if (MODE == SK_RESSQ) {
      ss = rows_sum(ss);
      if (g == 0) ssl[wave][r16] = ss;
      __syncthreads();
      if (threadIdx.x < M)
        p.ssq_out[(size_t)xb * M + threadIdx.x] =
            ((ssl[0][threadIdx.x] + ssl[1][threadIdx.x]) + ssl[2][threadIdx.x]) +
            ssl[3][threadIdx.x];
    }
  } else if (MODE == SK_SWIGLU) {
    const int n = xb * 32 + ta * 16 + 4 * g;
    if (owner && m < M && n < N) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = ya[j] / (1.0f + expf(-ya[j])) * yb2[j];
      store4(p.out, 1, (size_t)m * N + n, n, N, y);
    }
  } else {   // SK_ROPE
    const RopeArgs& r = p.rope;
    if (owner && m < M) {
      const int half = r.hd / 2;
      const int h = xb / p.nsub;
      const int i0 = (xb - h * p.nsub) * 32 + ta * 16 + 4 * g;
      int slot = r.row_slot ? r.row_slot[m] : m;
      if (slot < 0 || slot >= r.slot_cap) {
        set_status(r.status, EAGLE_DEV_BAD_INDEX);
        slot = -1;
      }
      float y1[4], y2[4];
      if (h < r.Hq + r.Hkv) {
        const double pos = (double)(r.pos_base + r.depth[m]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float cs, sn;
          rope_cs(pos, sinv[i0 + j], cs, sn);
          y1[j] = ya[j] * cs - yb2[j] * sn;
          y2[j] = yb2[j] * cs + ya[j] * sn;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y1[j] = ya[j];
          y2[j] = yb2[j];
        }
      }
      bf16_t* dst = nullptr;
      if (h < r.Hq) dst = r.q_out + ((size_t)m * r.Hq + h) * r.hd;
      else if (slot >= 0 && h < r.Hq + r.Hkv)
        dst = r.k_tree + ((size_t)(h - r.Hq) * r.ld_tree + slot) * r.hd;
      else if (slot >= 0)
        dst = r.v_tree + ((size_t)(h - r.Hq - r.Hkv) * r.ld_tree + slot) * r.hd;
      if (dst) {
        *(u32x2*)(dst + i0) = u32x2{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3])};
        *(u32x2*)(dst + i0 + half) =
            u32x2{pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3])};
      }
    }
  }
}

struct SkPlan {
  int nblk, S;
  size_t part_off, total;
};

// Column blocks by mode; k ranges per column block: the smallest power of two
// that puts >= 256 workgroups in flight (one per CU), with at least four k
// steps (one per wave) per workgroup.  (Measured on the Llama-3-8B draft
// round: 256 beats 512 and 128 - fewer hand-offs of partial tiles, yet every
// CU busy.)
static SkPlan sk_plan(int mode, int M, int K, int N, int heads, int hd) {
  SkPlan pl{};
  if (mode == SK_SWIGLU) pl.nblk = (N + 31) / 32;
  else if (mode == SK_ROPE) pl.nblk = heads * ((hd / 2) / 32);
  else pl.nblk = (N + 63) / 64;
  const int nk = K / kWsKG;
  int S = 1;
  while (S < kSkMaxS && pl.nblk * S < 256 && 2 * S <= nk / 4) S *= 2;
  // k ranges of at most 8 steps (two per wave, all in flight at once) when
  // one round of workgroups would otherwise hold more, for K <= 8192: the
  // draft's fuse product (K = 8192, 64 column blocks) then runs 512
  // workgroups, two per CU, in 17 instead of 20 us; longer K keeps fewer,
  // longer ranges (down: 25 against 24 us)
  if (pl.nblk * S <= 256 && nk <= 64)
    while (S < kSkMaxS && nk / S > 8) S *= 2;
  pl.S = S;
  pl.part_off = kSkCounterBytes;
  pl.total = pl.S > 1
                 ? pl.part_off + (((size_t)pl.S * pl.nblk * M * 64 * sizeof(float) + 255) & ~(size_t)255)
                 : 0;
  return pl;
}

template <int MODE>
static void launch_rows(SkParams p, const SkPlan& pl, void* ws, hipStream_t s) {
  p.nblk = pl.nblk;
  p.S = pl.S;
  char* w = (char*)ws;
  p.ctr = (int32_t*)w;
  p.part = w ? (float*)(w + pl.part_off) : nullptr;
  hipLaunchKernelGGL(linear_rows_kernel<MODE>, dim3(pl.nblk, pl.S), dim3(256), 0, s, p);
}

// Row runs for up to 64 activation rows when a workgroup's k range has at
// least kLinRrSteps steps (M = 64: the SwiGLU's 16 and 32 and the down
// projection's 7 steps run 7-11% faster that way; the 4-step o and qkv
// slices 1-15% slower).
constexpr int kLinRrSteps = 6;

// k slices for a projection: enough workgroups to fill the chip (about two per
// CU) while the fp32 partials stay below a quarter of the weight bytes; the
// count divides K / 128.
static int lin_ksplit(int M, int K, int N, int swiglu) {
  const int cols = lin_cols_block(lin_mt((M + 15) / 16, swiglu), swiglu);
  const int nblk = (N + cols - 1) / cols;
  const int nk = K / kWsKG;
  // SwiGLU with up to 64 rows and column blocks for most of the CUs: one
  // k slice, so no partials and no reduce launch (M = 64, N = 14336: 224
  // workgroups on row runs, 62 against 65 us with two slices and the reduce)
  if (swiglu && M <= 64 && 4 * nblk >= 3 * 256 && nk >= kLinRrSteps) return 1;
  const int want = (512 + nblk - 1) / nblk;
  int best = 1;
  for (int s = 1; s <= nk; ++s) {
    if (nk % s) continue;
    if (s > want) break;
    const double part = (double)s * (swiglu ? 2 : 1) * M * N * 4;
    const double wbytes = (double)(swiglu ? 2 : 1) * N * K * 2;
    if (s > 1 && part > 0.25 * wbytes) break;
    best = s;
  }
  return best;
}

// Workspace of the general path: the counter area (kept untouched, so one
// buffer can serve both paths) followed by the k-slice partials.
static size_t lin_workspace(int M, int K, int N, int swiglu) {
  if (M <= kSkMaxRows) return sk_plan(swiglu ? SK_SWIGLU : SK_PLAIN, M, K, N, 0, 0).total;
  const int s = lin_ksplit(M, K, N, swiglu);
  return s > 1 ? kSkCounterBytes + (size_t)s * (swiglu ? 2 : 1) * M * N * sizeof(float) : 0;
}

// Row-epilogue products (rmsnorm, deferred rmsnorm, rope): the largest layout
// any of them uses at this shape.
static size_t rows_workspace(int M, int K, int N) {
  size_t w = kSkCounterBytes + (size_t)lin_ksplit(M, K, N, 0) * M * N * sizeof(float);
  if (M <= kSkMaxRows) w = std::max(w, sk_plan(SK_PLAIN, M, K, N, 0, 0).total);
  return w;
}

static RowNorm row_norm(const float* ssq, int parts, int n, float eps) {
  return RowNorm{ssq, ssq ? parts : 0, n, eps};
}

static float* lin_partials(void* ws) { return (float*)((char*)ws + kSkCounterBytes); }

// lin_ksplit sizes the split from lin_mt((M + 15) / 16, ...) while the
// launches below round the row tiles up to 1, 2, 4, 8 or 16: both give the
// same W tiles for every M.
static_assert(lin_mt(3, 0) == lin_mt(4, 0) && lin_mt(5, 0) == lin_mt(8, 0) &&
                  lin_mt(9, 0) == lin_mt(16, 0) && lin_mt(3, 1) == lin_mt(4, 1) &&
                  lin_mt(5, 1) == lin_mt(8, 1) && lin_mt(9, 1) == lin_mt(16, 1),
              "row-tile buckets must not change the W tiling");

static bool lin_rr(const LinParams& p) {
  return p.M <= 64 && p.K / p.ksplit / kWsKG >= kLinRrSteps;
}

template <int NT, int SWIGLU>
static void launch_lin(const LinParams& p, hipStream_t s) {
  constexpr int MT = lin_mt(NT, SWIGLU);
  const int cols = lin_cols_block(MT, SWIGLU);
  const dim3 grid((p.N + cols - 1) / cols, p.ksplit);
  if (NT <= 4 && lin_rr(p))
    hipLaunchKernelGGL((linear_bf16_kernel<NT, SWIGLU, MT, NT <= 4>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((linear_bf16_kernel<NT, SWIGLU, MT, false>), grid, dim3(256), 0, s, p);
}

// GEMM only, writing fp32 partials (ksplit >= 1) for a row-wise epilogue.
static void launch_lin_partials(LinParams p, hipStream_t s) {
  p.to_part = 1;
  const int nt = (p.M + 15) / 16;
  if (nt <= 1) launch_lin<1, 0>(p, s);
  else if (nt <= 2) launch_lin<2, 0>(p, s);
  else if (nt <= 4) launch_lin<4, 0>(p, s);
  else if (nt <= 8) launch_lin<8, 0>(p, s);
  else launch_lin<16, 0>(p, s);
}

template <int SWIGLU>
static void dispatch_lin(LinParams p, hipStream_t s) {
  p.to_part = p.ksplit > 1 ? 1 : 0;
  const int nt = (p.M + 15) / 16;
  if (nt <= 1) launch_lin<1, SWIGLU>(p, s);
  else if (nt <= 2) launch_lin<2, SWIGLU>(p, s);
  else if (nt <= 4) launch_lin<4, SWIGLU>(p, s);
  else if (nt <= 8) launch_lin<8, SWIGLU>(p, s);
  else launch_lin<16, SWIGLU>(p, s);
  if (p.ksplit > 1) {
    const size_t MN = (size_t)p.M * p.N;
    hipLaunchKernelGGL(linear_reduce_kernel, dim3((unsigned)((MN + 1023) / 1024)), dim3(256), 0, s,
                       p, SWIGLU);
  }
}

}  // namespace eagle

using eagle::bf16_t;

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

extern "C" size_t eagle_linear_workspace(int32_t M, int32_t K, int32_t N, int32_t swiglu) {
  if (M < 1 || K < eagle::kWsKG || N < 1 || K % eagle::kWsKG) return 0;
  return eagle::lin_workspace(M, K, N, swiglu ? 1 : 0);
}

extern "C" int eagle_linear(const void* x, int32_t M, int32_t K, const void* W, int32_t N,
                            const float* residual, void* out, eagle_dtype out_dt,
                            void* workspace, size_t ws_bytes, hipStream_t stream) {
  EAGLE_REQUIRE(x && W && out, EAGLE_EINVAL);
  EAGLE_REQUIRE(M >= 1 && M <= EAGLE_MAX_TREE && K >= 1 && N >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(out_dt == EAGLE_BF16 || out_dt == EAGLE_F32, EAGLE_EINVAL);
  EAGLE_REQUIRE(K % eagle::kWsKG == 0, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(aligned16(x) && aligned16(W) && aligned16(out), EAGLE_EINVAL);
  const size_t need = eagle::lin_workspace(M, K, N, 0);
  EAGLE_REQUIRE(need == 0 || (workspace && aligned16(workspace)), EAGLE_EINVAL);
  EAGLE_REQUIRE(ws_bytes >= need, EAGLE_EWORKSPACE);
  if (M <= eagle::kSkMaxRows) {
    const eagle::SkPlan pl = eagle::sk_plan(eagle::SK_PLAIN, M, K, N, 0, 0);
    EAGLE_REQUIRE(pl.nblk <= eagle::kSkMaxBlocks, EAGLE_EUNSUPPORTED);
    eagle::SkParams p{};
    p.x = (const bf16_t*)x; p.M = M; p.K = K; p.w0 = (const bf16_t*)W; p.N = N;
    p.residual = residual; p.out = out; p.out_bf16 = out_dt == EAGLE_BF16 ? 1 : 0;
    eagle::launch_rows<eagle::SK_PLAIN>(p, pl, pl.total ? workspace : nullptr, stream);
    EAGLE_LAUNCH_CHECK();
    return EAGLE_OK;
  }
  const int ks = eagle::lin_ksplit(M, K, N, 0);
  eagle::LinParams p{(const bf16_t*)x, M, K, (const bf16_t*)W, nullptr, N, residual, out,
                     out_dt == EAGLE_BF16 ? 1 : 0, ks,
                     ks > 1 ? eagle::lin_partials(workspace) : nullptr};
  eagle::dispatch_lin<0>(p, stream);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_fuse3(const void* h_low, const void* h_mid, const void* h_high, int32_t M,
                           int32_t d, const void* W, int32_t N, void* out, eagle_dtype out_dt,
                           void* workspace, size_t ws_bytes, hipStream_t stream) {
  EAGLE_REQUIRE(h_low && h_mid && h_high && W && out, EAGLE_EINVAL);
  EAGLE_REQUIRE(M >= 1 && d >= 1 && N >= 1 && (int64_t)3 * d <= 0x7fffffff, EAGLE_EINVAL);
  EAGLE_REQUIRE(out_dt == EAGLE_BF16 || out_dt == EAGLE_F32, EAGLE_EINVAL);
  EAGLE_REQUIRE(M <= eagle::kSkMaxRows && d % eagle::kWsKG == 0, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(aligned16(h_low) && aligned16(h_mid) && aligned16(h_high) && aligned16(W) &&
                    aligned16(out), EAGLE_EINVAL);
  const int K = 3 * d;
  const size_t need = eagle::lin_workspace(M, K, N, 0);
  EAGLE_REQUIRE(need == 0 || (workspace && aligned16(workspace)), EAGLE_EINVAL);
  EAGLE_REQUIRE(ws_bytes >= need, EAGLE_EWORKSPACE);
  const eagle::SkPlan pl = eagle::sk_plan(eagle::SK_PLAIN, M, K, N, 0, 0);
  EAGLE_REQUIRE(pl.nblk <= eagle::kSkMaxBlocks, EAGLE_EUNSUPPORTED);
  eagle::SkParams p{};
  p.x = (const bf16_t*)h_low; p.M = M; p.K = K; p.w0 = (const bf16_t*)W; p.N = N;
  p.out = out; p.out_bf16 = out_dt == EAGLE_BF16 ? 1 : 0;
  p.xseg[0] = (const bf16_t*)h_low;
  p.xseg[1] = (const bf16_t*)h_mid;
  p.xseg[2] = (const bf16_t*)h_high;
  p.kseg = d;
  eagle::launch_rows<eagle::SK_PLAIN>(p, pl, pl.total ? workspace : nullptr, stream);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_linear_swiglu(const void* x, int32_t M, int32_t K, const float* in_ssq,
                                   int32_t in_parts, float in_eps, const void* w_gate,
                                   const void* w_up, int32_t N, void* out, void* workspace,
                                   size_t ws_bytes, hipStream_t stream) {
  EAGLE_REQUIRE(x && w_gate && w_up && out, EAGLE_EINVAL);
  EAGLE_REQUIRE(!in_ssq || (in_parts >= 1 && in_eps >= 0.0f), EAGLE_EINVAL);
  const eagle::RowNorm rn = eagle::row_norm(in_ssq, in_parts, K, in_eps);
  EAGLE_REQUIRE(M >= 1 && M <= EAGLE_MAX_TREE && K >= 1 && N >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(K % eagle::kWsKG == 0, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(aligned16(x) && aligned16(w_gate) && aligned16(w_up) && aligned16(out),
                EAGLE_EINVAL);
  const size_t need = eagle::lin_workspace(M, K, N, 1);
  EAGLE_REQUIRE(need == 0 || (workspace && aligned16(workspace)), EAGLE_EINVAL);
  EAGLE_REQUIRE(ws_bytes >= need, EAGLE_EWORKSPACE);
  if (M <= eagle::kSkMaxRows) {
    const eagle::SkPlan pl = eagle::sk_plan(eagle::SK_SWIGLU, M, K, N, 0, 0);
    EAGLE_REQUIRE(pl.nblk <= eagle::kSkMaxBlocks, EAGLE_EUNSUPPORTED);
    eagle::SkParams p{};
    p.x = (const bf16_t*)x; p.M = M; p.K = K; p.w0 = (const bf16_t*)w_gate;
    p.w1 = (const bf16_t*)w_up; p.N = N; p.out = out; p.out_bf16 = 1; p.in = rn;
    eagle::launch_rows<eagle::SK_SWIGLU>(p, pl, pl.total ? workspace : nullptr, stream);
    EAGLE_LAUNCH_CHECK();
    return EAGLE_OK;
  }
  const int ks = eagle::lin_ksplit(M, K, N, 1);
  eagle::LinParams p{(const bf16_t*)x, M, K, (const bf16_t*)w_gate, (const bf16_t*)w_up, N,
                     nullptr, out, 1, ks, ks > 1 ? eagle::lin_partials(workspace) : nullptr};
  p.in = rn;
  eagle::dispatch_lin<1>(p, stream);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_rmsnorm(const float* x, const float* gamma, int32_t M, int32_t N, float eps,
                             void* out, hipStream_t stream) {
  EAGLE_REQUIRE(x && gamma && out && M >= 1 && N >= 1 && eps >= 0.0f, EAGLE_EINVAL);
  hipLaunchKernelGGL(eagle::rmsnorm_kernel, dim3(M), dim3(256), 0, stream, x, gamma, N, eps,
                     (bf16_t*)out);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_rope_qkv(const float* qkv, int32_t M, int32_t Hq, int32_t Hkv, int32_t hd,
                              const int32_t* depth, int64_t pos_base, float theta,
                              const int32_t* row_slot, int32_t slot_cap, void* q_out,
                              void* k_tree, void* v_tree, int32_t ld_tree, int32_t* dev_status,
                              hipStream_t stream) {
  EAGLE_REQUIRE(qkv && depth && q_out && k_tree && v_tree, EAGLE_EINVAL);
  EAGLE_REQUIRE(M >= 1 && Hq >= 1 && Hkv >= 1 && hd >= 2 && hd % 2 == 0, EAGLE_EINVAL);
  EAGLE_REQUIRE(hd / 2 <= eagle::kRopeMaxHalf, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(slot_cap >= 1 && ld_tree >= slot_cap && theta > 0.0f && pos_base >= 0,
                EAGLE_EINVAL);
  eagle::RopeArgs r{Hq, Hkv, hd, depth, pos_base, (double)theta, row_slot, slot_cap,
                    (bf16_t*)q_out, (bf16_t*)k_tree, (bf16_t*)v_tree, ld_tree, dev_status};
  hipLaunchKernelGGL(eagle::rope_qkv_kernel, dim3(M), dim3(256), 0, stream, qkv, r);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" size_t eagle_linear_rows_workspace(int32_t M, int32_t K, int32_t N) {
  if (M < 1 || K < eagle::kWsKG || N < 1 || K % eagle::kWsKG) return 0;
  return eagle::rows_workspace(M, K, N);
}

extern "C" int eagle_linear_rmsnorm(const void* x, int32_t M, int32_t K, const void* W, int32_t N,
                                    const float* residual, float* out, const float* gamma,
                                    float eps, void* norm_out, void* workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  EAGLE_REQUIRE(x && W && out && gamma && norm_out && workspace, EAGLE_EINVAL);
  EAGLE_REQUIRE(M >= 1 && M <= EAGLE_MAX_TREE && K >= 1 && N >= 1 && eps >= 0.0f, EAGLE_EINVAL);
  EAGLE_REQUIRE(K % eagle::kWsKG == 0 && N % 4 == 0 && N <= eagle::kRowMaxN, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(aligned16(x) && aligned16(W) && aligned16(out) && aligned16(gamma) &&
                    aligned16(workspace) && (!residual || aligned16(residual)) &&
                    ((uintptr_t)norm_out & 7) == 0,
                EAGLE_EINVAL);
  EAGLE_REQUIRE(ws_bytes >= eagle_linear_rows_workspace(M, K, N), EAGLE_EWORKSPACE);
  eagle::LinParams p{(const bf16_t*)x, M, K, (const bf16_t*)W, nullptr, N, residual, out, 0,
                     eagle::lin_ksplit(M, K, N, 0), eagle::lin_partials(workspace)};
  p.ksplit = p.ksplit < 1 ? 1 : p.ksplit;
  eagle::launch_lin_partials(p, stream);
  hipLaunchKernelGGL(eagle::linear_reduce_norm_kernel, dim3(M), dim3(eagle::kRowThreads),
                     0, stream, p, gamma, eps, (bf16_t*)norm_out);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int32_t eagle_linear_norm_parts(int32_t M, int32_t K, int32_t N) {
  (void)K;
  if (M < 1 || N < 1) return 0;
  return M <= eagle::kSkMaxRows ? (N + 63) / 64 : (N + eagle::kRedCols - 1) / eagle::kRedCols;
}

extern "C" int eagle_linear_rmsnorm_deferred(const void* x, int32_t M, int32_t K, const void* W,
                                             int32_t N, const float* residual, float* out,
                                             const float* gamma, void* xg_out, float* ssq_out,
                                             void* workspace, size_t ws_bytes,
                                             hipStream_t stream) {
  EAGLE_REQUIRE(x && W && out && gamma && xg_out && ssq_out && workspace, EAGLE_EINVAL);
  EAGLE_REQUIRE(M >= 1 && M <= EAGLE_MAX_TREE && K >= 1 && N >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(K % eagle::kWsKG == 0 && N % 4 == 0 && N <= eagle::kRowMaxN, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(aligned16(x) && aligned16(W) && aligned16(out) && aligned16(gamma) &&
                    aligned16(workspace) && (!residual || aligned16(residual)) &&
                    ((uintptr_t)xg_out & 7) == 0 && ((uintptr_t)ssq_out & 3) == 0,
                EAGLE_EINVAL);
  EAGLE_REQUIRE(ws_bytes >= eagle_linear_rows_workspace(M, K, N), EAGLE_EWORKSPACE);
  if (M <= eagle::kSkMaxRows) {
    const eagle::SkPlan pl = eagle::sk_plan(eagle::SK_RESSQ, M, K, N, 0, 0);
    EAGLE_REQUIRE(pl.nblk <= eagle::kSkMaxBlocks, EAGLE_EUNSUPPORTED);
    eagle::SkParams p{};
    p.x = (const bf16_t*)x; p.M = M; p.K = K; p.w0 = (const bf16_t*)W; p.N = N;
    p.residual = residual; p.out = out; p.gamma = gamma; p.xg_out = (bf16_t*)xg_out;
    p.ssq_out = ssq_out;
    eagle::launch_rows<eagle::SK_RESSQ>(p, pl, workspace, stream);
    EAGLE_LAUNCH_CHECK();
    return EAGLE_OK;
  }
  eagle::LinParams p{(const bf16_t*)x, M, K, (const bf16_t*)W, nullptr, N, residual, out, 0,
                     eagle::lin_ksplit(M, K, N, 0), eagle::lin_partials(workspace)};
  p.ksplit = p.ksplit < 1 ? 1 : p.ksplit;
  eagle::launch_lin_partials(p, stream);
  hipLaunchKernelGGL(eagle::linear_reduce_dnorm_kernel,
                     dim3(M, (N + eagle::kRedCols - 1) / eagle::kRedCols), dim3(256), 0, stream, p,
                     gamma, (bf16_t*)xg_out, ssq_out);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_linear_rope_qkv(const void* x, int32_t M, int32_t K, const float* in_ssq,
                                     int32_t in_parts, float in_eps, const void* w_qkv,
                                     int32_t Hq, int32_t Hkv, int32_t hd, const int32_t* depth,
                                     int64_t pos_base, float theta, const int32_t* row_slot,
                                     int32_t slot_cap, void* q_out, void* k_tree, void* v_tree,
                                     int32_t ld_tree, void* workspace, size_t ws_bytes,
                                     int32_t* dev_status, hipStream_t stream) {
  EAGLE_REQUIRE(x && w_qkv && depth && q_out && k_tree && v_tree && workspace, EAGLE_EINVAL);
  EAGLE_REQUIRE(!in_ssq || (in_parts >= 1 && in_eps >= 0.0f), EAGLE_EINVAL);
  const eagle::RowNorm rn = eagle::row_norm(in_ssq, in_parts, K, in_eps);
  EAGLE_REQUIRE(M >= 1 && M <= EAGLE_MAX_TREE && K >= 1 && Hq >= 1 && Hkv >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(hd >= 8 && hd % 8 == 0 && hd / 2 <= eagle::kRopeMaxHalf, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(K % eagle::kWsKG == 0, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(slot_cap >= 1 && ld_tree >= slot_cap && theta > 0.0f && pos_base >= 0,
                EAGLE_EINVAL);
  const int N = (Hq + 2 * Hkv) * hd;
  EAGLE_REQUIRE((size_t)N * sizeof(float) <= 64 * 1024, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(aligned16(x) && aligned16(w_qkv) && aligned16(workspace), EAGLE_EINVAL);
  EAGLE_REQUIRE(ws_bytes >= eagle_linear_rows_workspace(M, K, N), EAGLE_EWORKSPACE);
  eagle::RopeArgs r{Hq, Hkv, hd, depth, pos_base, (double)theta, row_slot, slot_cap,
                    (bf16_t*)q_out, (bf16_t*)k_tree, (bf16_t*)v_tree, ld_tree, dev_status};
  if (M <= eagle::kSkMaxRows && hd % 64 == 0 && ((uintptr_t)q_out & 7) == 0 &&
      ((uintptr_t)k_tree & 7) == 0 && ((uintptr_t)v_tree & 7) == 0) {
    const eagle::SkPlan pl = eagle::sk_plan(eagle::SK_ROPE, M, K, N, Hq + 2 * Hkv, hd);
    EAGLE_REQUIRE(pl.nblk <= eagle::kSkMaxBlocks, EAGLE_EUNSUPPORTED);
    eagle::SkParams p{};
    p.x = (const bf16_t*)x; p.M = M; p.K = K; p.w0 = (const bf16_t*)w_qkv; p.N = N;
    p.nsub = (hd / 2) / 32;
    p.rope = r;
    p.in = rn;
    eagle::launch_rows<eagle::SK_ROPE>(p, pl, workspace, stream);
    EAGLE_LAUNCH_CHECK();
    return EAGLE_OK;
  }
  eagle::LinParams p{(const bf16_t*)x, M, K, (const bf16_t*)w_qkv, nullptr, N, nullptr, nullptr,
                     0, eagle::lin_ksplit(M, K, N, 0), eagle::lin_partials(workspace)};
  p.in = rn;
  eagle::launch_lin_partials(p, stream);
  const int H = Hq + 2 * Hkv;
  hipLaunchKernelGGL(eagle::linear_reduce_rope_kernel,
                     dim3(M, (H + eagle::kRopeHeads - 1) / eagle::kRopeHeads), dim3(256),
                     (size_t)eagle::kRopeHeads * hd * sizeof(float), stream, p, r);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_draft_prepare(const int32_t* frontier, int32_t kf, const int32_t* pool_token,
                                   const int32_t* pool_parent, const int32_t* pool_depth,
                                   int32_t pool_n, int32_t* slot_of_pool, int32_t slot_base,
                                   int32_t slot_cap, int32_t* slot_parent, uint64_t* slot_mask,
                                   int32_t words, int32_t* row_token, int32_t* row_depth,
                                   int32_t* row_slot, int32_t* row_src, const float* feat,
                                   const float* root_feat, const void* embed, int32_t V,
                                   int32_t d, void* x_in, int32_t* dev_status,
                                   hipStream_t stream) {
  EAGLE_REQUIRE(frontier && pool_token && pool_parent && pool_depth && slot_of_pool &&
                    slot_parent && row_token && row_depth && row_slot && row_src,
                EAGLE_EINVAL);
  EAGLE_REQUIRE(kf >= 1 && kf <= EAGLE_MAX_TREE && pool_n >= 1 && V >= 1, EAGLE_EINVAL);
  EAGLE_REQUIRE(slot_base >= 0 && slot_base + kf <= slot_cap, EAGLE_EINVAL);
  EAGLE_REQUIRE(!slot_mask || (words >= (slot_cap + 63) / 64 && words <= 4), EAGLE_EINVAL);
  EAGLE_REQUIRE(!x_in || (feat && root_feat && embed && d >= 1), EAGLE_EINVAL);
  hipLaunchKernelGGL(eagle::draft_prepare_kernel, dim3(kf), dim3(256), 0, stream, frontier,
                     pool_token, pool_parent, pool_depth, pool_n, slot_of_pool, slot_base,
                     slot_cap, slot_parent, slot_mask, words, row_token, row_depth, row_slot,
                     row_src, feat, root_feat, (const bf16_t*)embed, V, d, (bf16_t*)x_in,
                     dev_status);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_embed_deferred(int32_t M, const int32_t* token, const void* embed,
                                    int32_t V, int32_t d, const float* gamma, float* out,
                                    void* xg_out, float* ssq_out, int32_t* dev_status,
                                    hipStream_t stream) {
  EAGLE_REQUIRE(token && embed && gamma && out && xg_out && ssq_out && M >= 1 && V >= 1 && d >= 1,
                EAGLE_EINVAL);
  EAGLE_REQUIRE(d % 8 == 0, EAGLE_EUNSUPPORTED);
  EAGLE_REQUIRE(aligned16(embed) && aligned16(gamma) && aligned16(out) && aligned16(xg_out),
                EAGLE_EINVAL);
  hipLaunchKernelGGL(eagle::embed_deferred_kernel, dim3(M), dim3(256), 0, stream, token,
                     (const bf16_t*)embed, V, d, gamma, out, (bf16_t*)xg_out, ssq_out,
                     dev_status);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}

extern "C" int eagle_embed(int32_t M, const int32_t* token, const void* embed, int32_t V,
                           int32_t d, float* out, int32_t* dev_status, hipStream_t stream) {
  EAGLE_REQUIRE(token && embed && out && M >= 1 && V >= 1 && d >= 1, EAGLE_EINVAL);
  hipLaunchKernelGGL(eagle::embed_kernel, dim3(M), dim3(256), 0, stream, token,
                     (const bf16_t*)embed, V, d, out, dev_status);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
