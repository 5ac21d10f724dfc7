// Weight-streaming bf16 MFMA core shared by the LM head and the decoder-layer
// projections: Y[m][n] = sum_k X[m][k] W[n][k] for few rows m (<= 256) and many
// weight rows n.
//
// With few activation rows every weight byte is used <= 256 times, so these
// products are bound by reading W from HBM once.  A 4-wave workgroup owns
// 4 x MT x 16 weight rows; each wave issues its W rows' 16-byte loads for the
// next 128-wide k step before running the MFMAs of the current one (the small
// activation loads are issued first, so staging them in LDS never waits for
// the weight loads still in flight).  W rows are
// the MFMA M dimension (v_mfma_f32_16x16x32_bf16 A operand, straight from
// registers) and the activation rows are N, staged per k step in LDS
// (double-buffered; rows padded by 16 bytes so the 16 lanes of one b128 read
// land on distinct banks).  MFMA i of a 128-wide k step covers k = 32i..32i+31
// with lane group g (lanes 16g..16g+15) holding k = 32i + 8g..+7, so in every
// 16-byte load instruction the four lanes of a W row read 64 contiguous bytes
// (16 rows x 64 bytes per instruction).
//
// After run(), lane (g = lane / 16, r16 = lane % 16) of a wave holds, for tile
// (mt, nt), Y[m = 16 nt + r16][n = n(mt) + 4 g + j] in acc[mt][nt][j], where n(mt)
// is the first weight row of the wave's M tile mt.
#pragma once

#include "common.h"

namespace eagle {

constexpr int kWsKG = 128;        // k elements per step
constexpr int kWsLds = kWsKG + 8;  // padded LDS row (bf16 elements)

template <int NT>
constexpr int ws_lds_elems() {
  return 2 * 16 * NT * kWsLds;
}

__device__ __forceinline__ bf16x8 ws_as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// wrow[mt]: pointer to the weight row of this lane for tile mt, already offset
// by 8 g elements.  X: [M][ldx] bf16 activations (rows >= M read as zero).
// fs: LDS scratch of ws_lds_elems<NT>() elements.  K % 128 == 0.
template <int NT, int MT>
__device__ __forceinline__ void wstream_mfma(const bf16_t* const (&wrow)[MT], const bf16_t* X,
                                             int ldx, int M, int K, bf16_t* fs,
                                             f32x4 (&acc)[MT][NT]) {
  constexpr int TP = 16 * NT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  bf16_t* fs0 = fs;
  bf16_t* fs1 = fs + TP * kWsLds;

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_x = [&](int kk, u32x4 (&fr)[NT]) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int c = tid + 256 * j;
      const int row = c >> 4;
      const int col = (c & 15) * 8;
      fr[j] = row < M ? *(const u32x4*)(X + (size_t)row * ldx + kk * kWsKG + col)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_x = [&](bf16_t* buf, const u32x4 (&fr)[NT]) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int c = tid + 256 * j;
      *(u32x4*)(&buf[(c >> 4) * kWsLds + (c & 15) * 8]) = fr[j];
    }
  };
  auto load_w = [&](int kk, u32x4 (&wr)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[mt][i] = *(const u32x4*)(wrow[mt] + kk * kWsKG + i * 32);
  };
  auto compute = [&](const bf16_t* fb, const u32x4 (&wr)[MT][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8 b[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        b[nt] = *(const bf16x8*)(fb + (nt * 16 + r16) * kWsLds + i * 32 + g * 8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = ws_as_bf16x8(wr[mt][i]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nt], acc[mt][nt], 0, 0, 0);
      }
    }
  };

  const int nk = K / kWsKG;
  u32x4 wa[MT][4], wb[MT][4];
  u32x4 fr[NT];
  load_x(0, fr);
  store_x(fs0, fr);
  load_w(0, wa);
  __syncthreads();
  for (int kk = 0; kk < nk; kk += 2) {
    const bool more1 = kk + 1 < nk;
    if (more1) {
      load_x(kk + 1, fr);   // first: the LDS store below waits only for these
      load_w(kk + 1, wb);
    }
    compute(fs0, wa);
    if (more1) store_x(fs1, fr);
    __syncthreads();
    if (!more1) break;
    const bool more2 = kk + 2 < nk;
    if (more2) {
      load_x(kk + 2, fr);
      load_w(kk + 2, wa);
    }
    compute(fs1, wb);
    if (more2) store_x(fs0, fr);
    __syncthreads();
  }
}


// Row-run variant: each 16-byte load instruction of a wave covers 4 weight
// rows x 256 contiguous bytes (lane l: row 4 i + l / 16 of the tile, bytes
// 16 (l % 16) of the k step), issued with the non-temporal policy; the wave
// then passes the step through a private LDS tile (rows of 256 bytes, 16-byte
// chunks XOR-swizzled by row so that both the writes and the operand reads
// touch 64 distinct banks per 16 lanes) to reach the MFMA operand layout.
// tile_row0[mt]: first weight row of tile mt (rows past nrows read zero: each
// tile has its own buffer range, so offsets stay small at any matrix size);
// wsel[mt]: 0 -> matrix w0, 1 -> w1; nrows rows of ldw elements per matrix,
// w0 / w1 / X pointing at the first k of the range (K wide, K % 128 == 0).
// wl: MT x 4 KB of LDS private to the wave.
constexpr int kNtPolicy = 1 << 1;    // buffer cache policy bit: nt

// XSINGLE: one activation buffer instead of two (half the LDS; one more
// barrier per k step).
template <int NT, int MT, bool XSINGLE = false>
__device__ __forceinline__ void wstream_mfma_rr(const bf16_t* w0, const bf16_t* w1, int nrows,
                                                int ldw, const int (&tile_row0)[MT],
                                                const int (&wsel)[MT], const bf16_t* X, int ldx,
                                                int M, int K, bf16_t* fs, char* wl,
                                                f32x4 (&acc)[MT][NT]) {
  constexpr int TP = 16 * NT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int r16 = lane & 15;
  bf16_t* fs0 = fs;
  bf16_t* fs1 = fs + TP * kWsLds;
  __amdgpu_buffer_rsrc_t trs[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int rows = max(0, min(16, nrows - tile_row0[mt]));
    trs[mt] = buf_rsrc_uniform((wsel[mt] ? w1 : w0) + (size_t)tile_row0[mt] * ldw,
                               (size_t)rows * ldw * sizeof(bf16_t));
  }
  // byte offset of this lane's run in instruction 0 of a tile; instruction i
  // adds 4 i rows, step kk adds 256 kk bytes
  const uint32_t voff = (uint32_t)(g * ldw * sizeof(bf16_t)) + r16 * 16;
  const uint32_t istride = 4u * ldw * sizeof(bf16_t);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_x = [&](int kk, u32x4 (&fr)[NT]) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int c = tid + 256 * j;
      const int row = c >> 4;
      const int col = (c & 15) * 8;
      fr[j] = row < M ? *(const u32x4*)(X + (size_t)row * ldx + kk * kWsKG + col)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_x = [&](bf16_t* buf, const u32x4 (&fr)[NT]) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int c = tid + 256 * j;
      *(u32x4*)(&buf[(c >> 4) * kWsLds + (c & 15) * 8]) = fr[j];
    }
  };
  auto load_w = [&](int kk, u32x4 (&wr)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wr[mt][i] = __builtin_amdgcn_raw_buffer_load_b128(trs[mt], voff,
                                                          (uint32_t)(i * istride + kk * 256),
                                                          kNtPolicy);
  };
  // instruction i's lane l holds row 4 i + g, chunk r16
  auto put_w = [&](const u32x4 (&wr)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + g;
        *(u32x4*)(wl + mt * 4096 + row * 256 + ((r16 ^ row) << 4)) = wr[mt][i];
      }
  };
  auto compute = [&](const bf16_t* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x8 b[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        b[nt] = *(const bf16x8*)(fb + (nt * 16 + r16) * kWsLds + i * 32 + g * 8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = *(const bf16x8*)(wl + mt * 4096 + r16 * 256 + (((4 * i + g) ^ r16) << 4));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nt], acc[mt][nt], 0, 0, 0);
      }
    }
  };

  const int nk = K / kWsKG;
  u32x4 wr[MT][4];
  u32x4 fr[NT];
  load_x(0, fr);
  load_w(0, wr);
  store_x(fs0, fr);
  put_w(wr);
  __syncthreads();
  for (int kk = 0; kk < nk; ++kk) {
    const bool more = kk + 1 < nk;
    if (more) {
      load_x(kk + 1, fr);
      load_w(kk + 1, wr);
    }
    if (XSINGLE) {
      compute(fs0);
      __syncthreads();   // every wave is done with step kk's activations
      if (more) {
        store_x(fs0, fr);
        put_w(wr);
      }
    } else {
      compute((kk & 1) ? fs1 : fs0);
      if (more) {
        store_x((kk & 1) ? fs0 : fs1, fr);
        put_w(wr);     // (after this wave's operand reads of step kk: LDS keeps a wave's order)
      }
    }
    __syncthreads();
  }
}

}  // namespace eagle
