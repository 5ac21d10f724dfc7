// Ancestor bitmask of a draft tree.
//
// Source: "EAGLE-2: Feature-Level Speculative Decoding Guide", Key
// Architectural Mechanics 3 - tokens attend to their ancestors and never to
// another branch; a node sees itself (the chain case is causal attention).
//
// One thread per node walks up through its parents.  Every step checks that
// the parent precedes the node it hangs from, so each walk strictly decreases
// and ends within T steps even on bad input.  T <= 256 keeps the whole job in
// one workgroup; the mask (<= 8 KB) is written with one 8-byte store per word.
#include "common.h"

namespace eagle {

__global__ __launch_bounds__(256) void build_tree_mask_kernel(
    const int32_t* __restrict__ parents, int T, int words, uint64_t* __restrict__ mask,
    int32_t* __restrict__ depth, int32_t* __restrict__ status) {
  __shared__ int32_t par[EAGLE_MAX_TREE];
  for (int i = threadIdx.x; i < T; i += blockDim.x) par[i] = parents[i];
  __syncthreads();
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    uint64_t m[4] = {0, 0, 0, 0};
    m[i >> 6] |= 1ull << (i & 63);
    int j = i;
    int d = 0;
    int p = par[i];
    while (p != -1) {
      if (p < 0 || p >= j) {
        set_status(status, EAGLE_DEV_BAD_PARENT);
        break;
      }
      m[p >> 6] |= 1ull << (p & 63);
      ++d;
      j = p;
      p = par[p];
    }
    for (int w = 0; w < words; ++w) mask[(size_t)i * words + w] = w < 4 ? m[w] : 0ull;
    depth[i] = d;
  }
}

}  // namespace eagle

extern "C" int eagle_build_tree_mask(const int32_t* parents, int32_t T, int32_t words,
                                     uint64_t* mask, int32_t* depth, int32_t* dev_status,
                                     hipStream_t stream) {
  EAGLE_REQUIRE(parents && mask && depth, EAGLE_EINVAL);
  EAGLE_REQUIRE(T >= 1 && T <= EAGLE_MAX_TREE, EAGLE_EINVAL);
  EAGLE_REQUIRE(words >= (T + 63) / 64 && words <= 4, EAGLE_EINVAL);
  EAGLE_REQUIRE(((uintptr_t)mask & 7) == 0, EAGLE_EINVAL);
  hipLaunchKernelGGL(eagle::build_tree_mask_kernel, dim3(1), dim3(256), 0, stream, parents, T,
                     words, mask, depth, dev_status);
  EAGLE_LAUNCH_CHECK();
  return EAGLE_OK;
}
