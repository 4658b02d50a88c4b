// Sequence-tiled SwiGLU MLP, element-wise parts ("Road to 5 Million Tokens"
// talk summary, Chapters: the sequence-tiling chapter -- the MLP is computed
// in pieces along the sequence so that its S-long intermediates, here the
// [S, F] gate, up and activation tensors, never exist at once). The GEMMs
// around them are gemm_bf16.hpp's; these kernels work on one tile's [tile][F]
// buffers:
//   forward:  a = silu(g) * u                        (g = x Wg^T, u = x Wu^T)
//   backward: du = da * silu(g),  dg = da * u * silu'(g),
//             silu(g) = g s(g), silu'(g) = s(g) (1 + g (1 - s(g))), s = sigmoid.
// Rows T <= r < tile (past the last token of a ragged tile) are written as
// zeros, because the weight-gradient GEMMs read whole 64-row K steps.
#pragma once

#include "common.hpp"

namespace upipe {

__device__ __forceinline__ float sigmoidf_(float g) { return 1.f / (1.f + __expf(-g)); }

// a[r][j] = bf16(silu(g) u) for r < T, 0 for T <= r < gridDim.x; 8 elements
// (16 bytes of bf16) per thread and step. F is a multiple of 8.
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const bf16* __restrict__ g, const bf16* __restrict__ u,
                                                        bf16* __restrict__ a, int T, int F) {
  const int r = blockIdx.x;
  const size_t row = (size_t)r * F;
  for (int j = threadIdx.x * 8; j < F; j += 256 * 8) {
    bf16x8 out;
    if (r < T) {
      const bf16x8 gv = *reinterpret_cast<const bf16x8*>(g + row + j);
      const bf16x8 uv = *reinterpret_cast<const bf16x8*>(u + row + j);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gf = (float)gv[e];
        out[e] = (bf16)(gf * sigmoidf_(gf) * (float)uv[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = (bf16)0.f;
    }
    *reinterpret_cast<bf16x8*>(a + row + j) = out;
  }
}

// From da (fp32 [tile][F]) and the tile's g and u (bf16), overwrite g with
// dg and u with du (bf16), each element read and written by one thread; rows
// past T become zero.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ da, bf16* __restrict__ g,
                                                        bf16* __restrict__ u, int T, int F) {
  const int r = blockIdx.x;
  const size_t row = (size_t)r * F;
  for (int j = threadIdx.x * 8; j < F; j += 256 * 8) {
    bf16x8 dg, du;
    if (r < T) {
      const bf16x8 gv = *reinterpret_cast<const bf16x8*>(g + row + j);
      const bf16x8 uv = *reinterpret_cast<const bf16x8*>(u + row + j);
      const floatx4 d0 = *reinterpret_cast<const floatx4*>(da + row + j);
      const floatx4 d1 = *reinterpret_cast<const floatx4*>(da + row + j + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = e < 4 ? d0[e] : d1[e - 4];
        const float gf = (float)gv[e], uf = (float)uv[e];
        const float sg = sigmoidf_(gf);
        du[e] = (bf16)(d * gf * sg);
        dg[e] = (bf16)(d * uf * sg * (1.f + gf * (1.f - sg)));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dg[e] = du[e] = (bf16)0.f;
    }
    *reinterpret_cast<bf16x8*>(g + row + j) = dg;
    *reinterpret_cast<bf16x8*>(u + row + j) = du;
  }
}

}  // namespace upipe
