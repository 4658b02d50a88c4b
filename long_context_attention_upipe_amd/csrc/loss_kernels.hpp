// Sequence-tiled cross-entropy over the vocabulary ("Road to 5 Million
// Tokens" talk summary, Chapters: the sequence-tiling chapter -- the loss
// and the MLP are computed in pieces along the sequence so that their
// S-long intermediates never exist at once; talk digest, Tips: tile the
// element-wise parts along the sequence). The logits of one tile of tokens
// live in a bounded [tile, V] buffer; this kernel turns each of its rows
// into the token's loss and, for the backward, the row of
//   G = dloss/dlogits = scale * (softmax(z) - onehot(label))
// that the two GEMMs of the backward consume.
#pragma once

#include "common.hpp"

namespace upipe {

// Combine two (max, sum of exp(x - max)) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -__builtin_inff()) return;  // both empty
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

// One 256-thread workgroup per row of the tile. Row r < T: logits z = row r
// of `logits` (V fp32 values, row stride ldl); writes loss[r] = lse(z) -
// z[label] (natural log; 0 for a label < 0, which is ignored) and, when G is
// set, G[r][j] = bf16(scale * (exp(z_j - lse) - [j == label])) for j < V and
// 0 for V <= j < ldg (0 across the row for an ignored label). A label >= V
// names no logit: nothing is read for it, and the row's loss and its G
// values j < V are NaN, so the error shows in loss, dh and dW. Rows T <= r <
// gridDim.x write a zero G row (the backward GEMMs read whole 64-row tiles).
// The reduction order is fixed, so results are deterministic.
__global__ __launch_bounds__(256) void ce_rows_kernel(const float* __restrict__ logits, int ldl,
                                                     const int32_t* __restrict__ labels, float* __restrict__ loss,
                                                     bf16* __restrict__ G, int ldg, int T, int V, float scale) {
  __shared__ float red_m[4], red_s[4];
  __shared__ float s_lse;
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bf16* g = G ? G + (size_t)r * ldg : nullptr;
  if (r >= T) {
    for (int j = tid * 8; j < ldg; j += 256 * 8) *reinterpret_cast<uint4*>(g + j) = make_uint4(0, 0, 0, 0);
    return;
  }
  const float* z = logits + (size_t)r * ldl;
  const int label = labels[r];
  const bool bad_label = label >= V;
  // pass 1: per-thread online (max, sum) over 4-wide slices, then the waves, then the workgroup
  float m = -__builtin_inff(), s = 0.f;
  for (int j = tid * 4; j < V; j += 256 * 4) {
    const floatx4 x = *reinterpret_cast<const floatx4*>(z + j);
    const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    const float ss = __expf(x[0] - mx) + __expf(x[1] - mx) + __expf(x[2] - mx) + __expf(x[3] - mx);
    lse_merge(m, s, mx, ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) {
    red_m[wave] = m;
    red_s[wave] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float mm = red_m[0], sm = red_s[0];
    for (int w = 1; w < 4; ++w) lse_merge(mm, sm, red_m[w], red_s[w]);
    const float lse = mm + __logf(sm);
    s_lse = lse;
    loss[r] = bad_label ? __builtin_nanf("") : label >= 0 ? lse - z[label] : 0.f;
  }
  __syncthreads();
  if (!g) return;
  const float lse = s_lse;
  const float sc = bad_label ? __builtin_nanf("") : label >= 0 ? scale : 0.f;
  // pass 2: the gradient row, 8 values (16 bytes of bf16) per thread and step
  for (int j = tid * 8; j < ldg; j += 256 * 8) {
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = j + e;
      float v = 0.f;
      if (c < V) v = sc * (__expf(z[c] - lse) - (c == label ? 1.f : 0.f));
      out[e] = (bf16)v;
    }
    *reinterpret_cast<bf16x8*>(g + j) = out;
  }
}

}  // namespace upipe
