// HBM-bound helper kernels around the attention kernels.
//
//  * pack / unpack: move a head chunk between the caller's token-major
//    [S, H, d] tensors and the pool's head-major [hc, S, d] buffers. On one
//    GPU this copy stands in for the Ulysses all-to-all that would bring the
//    chunk's heads, over the whole sequence, into the reused buffer
//    ("Road to 5 Million Tokens" talk summary, Chapters: Ulysses exchanges
//    activations between GPUs; batched heads reuse the previous batch's
//    buffer).
//  * bwd_pre: -D_i = -<dO_i, O_i> per row in fp32 from the stored output
//    (plus its stored rounding residual when there is one; stored negated so
//    the dK/dV kernel can start its dP accumulator from it), the
//    chunk's dO rows packed, and lse_i * log2(e) (the base-2 exponent offset
//    the backward kernels use), all in one pass;
//  * tail_rows: a zero-padded copy of a matrix's last rows.
#pragma once

#include "common.hpp"

namespace upipe {

// Grid-stride loops of the copy kernels run over tokens with a 64-bit index
// (S * nh * vpr can exceed 2^32 at multi-million-token lengths, where a 32-bit
// grid-stride index would wrap and never end); each block iteration covers
// max(1, 256 / per) whole tokens of per = nh * vpr vectors, so the divisions
// inside a token stay 32-bit and small.

// dst[hl][i][:] = src[i][h0 + hl][:]  (vpr = 16-byte vectors per row).
__global__ __launch_bounds__(256) void pack_heads_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        int S, int H, int h0, int nh, int vpr) {
  const int per = nh * vpr;
  const int tpi = max(1, 256 / per);  // tokens per block iteration
  for (int64_t t0 = (int64_t)blockIdx.x * tpi; t0 < S; t0 += (int64_t)gridDim.x * tpi) {
    for (int e = threadIdx.x; e < tpi * per; e += 256) {
      const int64_t i = t0 + e / per;
      if (i >= S) break;
      const int rem = e % per;
      const int hl = rem / vpr, v = rem % vpr;
      dst[((size_t)hl * S + i) * vpr + v] = src[((size_t)i * H + h0 + hl) * vpr + v];
    }
  }
}

// dst[i][h0 + hl][:] = src[hl][i][:]
__global__ __launch_bounds__(256) void unpack_heads_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          int S, int H, int h0, int nh, int vpr) {
  const int per = nh * vpr;
  const int tpi = max(1, 256 / per);
  for (int64_t t0 = (int64_t)blockIdx.x * tpi; t0 < S; t0 += (int64_t)gridDim.x * tpi) {
    for (int e = threadIdx.x; e < tpi * per; e += 256) {
      const int64_t i = t0 + e / per;
      if (i >= S) break;
      const int rem = e % per;
      const int hl = rem / vpr, v = rem % vpr;
      dst[((size_t)i * H + h0 + hl) * vpr + v] = src[((size_t)hl * S + i) * vpr + v];
    }
  }
}

// Transposed pack of bf16 V heads for the forward kernel, whose only use of V
// is as the operand of O^T += V^T P^T, contracting over keys. Keys go in
// blocks of 64; block b of head hl is a contiguous [D][64] matrix
//   dst[hl][b][c][p] = src[64b + j(p)][h0 + hl][c],  p < 64,
// with j(p) = (p & ~15) | perm16(p & 15): inside each group of 16 keys the
// positions follow the key order of a P fragment taken from score registers,
// so the 8 keys one lane contributes to an MFMA step sit in 16 consecutive
// bytes of a row. Keys >= S hold 0 (the last block is padded). Blocks are
// contiguous so that a key tile is one 16 KiB (d = 128) run of memory, not D
// rows a whole sequence apart. One workgroup moves one block through LDS.
template <int D>
__global__ __launch_bounds__(256) void pack_vt_kernel(const bf16* __restrict__ src, bf16* __restrict__ dst, int S,
                                                     int Sp, int H, int h0) {
  constexpr int VPR = D / 8;  // 16-byte vectors per key row
  __shared__ __attribute__((aligned(16))) bf16 t[64][D + 8];
  const int kb = blockIdx.x, hl = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < 64 * VPR; i += 256) {
    const int r = i / VPR, v = i % VPR;
    const int key = kb * 64 + r;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (key < S) x = *reinterpret_cast<const uint4*>(src + ((size_t)key * H + h0 + hl) * D + v * 8);
    *reinterpret_cast<uint4*>(&t[r][v * 8]) = x;
  }
  __syncthreads();
  for (int i = tid; i < D * 8; i += 256) {
    const int c = i / 8, pv = i % 8;
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = pv * 8 + e;
      y[e] = t[(pos & ~15) | perm16(pos & 15)][c];
    }
    *reinterpret_cast<bf16x8*>(dst + (size_t)hl * D * Sp + ((size_t)kb * D + c) * 64 + pv * 8) = y;
  }
}

// Where bwd_pre finds the chunk's rows: element e of head hl at token i is
// p[i * tok + hl * head + e] (the caller's token-major [S, H, d] at head h0:
// tok = H*d, head = d; a head-major pool buffer [hc][S][d]: tok = d,
// head = S*d).
template <typename T>
struct RowsView {
  const T* p;
  int64_t tok, head;
};

// One group of D/EPV lanes per (row, head): reads a 16-byte slice of out and
// dout each, copies the dout slice into the pool (if dout_pool is set),
// reduces the dot product. lse: the chunk's natural-log rows, head stride S.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(RowsView<T> out, RowsView<T> out_lo, RowsView<T> dout,
                                                     const float* __restrict__ lse, T* __restrict__ dout_pool,
                                                     float* __restrict__ negD, float* __restrict__ lse2, int S,
                                                     int nh) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int TPR = D / EPV;  // lanes per row: 16 (bf16, d=128), 8, 16 or 32
  constexpr int RPB = 256 / TPR;
  const int sub = threadIdx.x % TPR;
  // Row slots of one block iteration: whole tokens, max(1, RPB / nh) of them,
  // with a 64-bit token index (see the copy kernels above).
  const int tpi = max(1, RPB / nh);
  for (int64_t t0 = (int64_t)blockIdx.x * tpi; t0 < S; t0 += (int64_t)gridDim.x * tpi)
  for (int slot = threadIdx.x / TPR; slot < tpi * nh; slot += RPB) {
    const int64_t i = t0 + slot / nh;
    if (i >= S) break;
    const int hl = slot % nh;
    const int e0 = sub * EPV;
    const uint4 ov = *reinterpret_cast<const uint4*>(out.p + i * out.tok + hl * out.head + e0);
    const uint4 dv = *reinterpret_cast<const uint4*>(dout.p + i * dout.tok + hl * dout.head + e0);
    if (dout_pool) *reinterpret_cast<uint4*>(dout_pool + ((size_t)hl * S + i) * D + e0) = dv;
    const uint4 lv = out_lo.p ? *reinterpret_cast<const uint4*>(out_lo.p + i * out_lo.tok + hl * out_lo.head + e0)
                              : uint4{0, 0, 0, 0};
    const T* oe = reinterpret_cast<const T*>(&ov);
    const T* le = reinterpret_cast<const T*>(&lv);
    const T* de = reinterpret_cast<const T*>(&dv);
    float acc = 0.f;
    // out + out_lo is exact in fp32 (two 8-bit-mantissa parts, 2^-9 apart)
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc = fmaf(to_f32(oe[e]) + to_f32(le[e]), to_f32(de[e]), acc);
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (sub == 0) {
      negD[(size_t)hl * S + i] = -acc;
      lse2[(size_t)hl * S + i] = lse[(size_t)hl * S + i] * kLog2e;
    }
  }
}

// dst [64][Dm] = rows 0 .. valid-1 of src [.][Dm], then zero rows: the last,
// partial 64-deep K step of a GEMM that contracts over tokens (one operand
// zero past the sequence end). One workgroup per row; Dm a multiple of 8.
__global__ __launch_bounds__(256) void tail_rows_kernel(const bf16* __restrict__ src, bf16* __restrict__ dst,
                                                       int valid, int Dm) {
  const int r = blockIdx.x;
  for (int j = threadIdx.x * 8; j < Dm; j += 256 * 8) {
    const uint4 v = r < valid ? *reinterpret_cast<const uint4*>(src + (size_t)r * Dm + j) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(dst + (size_t)r * Dm + j) = v;
  }
}

}  // namespace upipe
