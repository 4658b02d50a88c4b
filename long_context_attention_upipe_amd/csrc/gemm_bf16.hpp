// bf16 GEMM with fp32 accumulation on gfx950 MFMA, for the projections that
// the chunked attention block runs around each head chunk (q, k, v of the
// chunk's heads from the layer input, and the chunk's share of the output
// projection), so that no tensor of every head over the whole sequence is
// formed ("Road to 5 Million Tokens" talk summary, Chapters: the Q&A on which
// tensors the head batching targets, the layer's Q, K and V).
//
//   C[M, N] = A[M, K] B[K, N]      (or C += ..., fp32 C only)
//
// Operands are addressed through a layout descriptor: each one is stored
// with either its K index contiguous ("k-major", e.g. a token-major
// activation [M][K] or a torch Linear weight [N][K]) or its M / N index
// contiguous ("mn-major", [K][M] or [K][N]). The contiguous index may run in
// blocks (a head-major [heads][S][d] buffer read as one [S][heads*d] matrix).
// Tiles go global -> LDS directly (global_load_lds), double-buffered. Both
// operand kinds are read in one k order: a P-fragment order in which the 8
// values a lane supplies for a 16-deep MFMA step are k = 4h..4h+3 and
// 8+4h..8+4h+3 (h = lane half); mn-major tiles give that order with the
// transposed LDS read, k-major tiles with two 8-byte reads. So any pair of
// layouts feeds v_mfma_f32_32x32x16_bf16 without a transposing copy. When
// both operands are k-major they use the plain order instead, one 16-byte
// LDS read per fragment.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "lds_tiles.hpp"

namespace upipe {

// Element (c, o) of an operand, c its contiguous index (K for k-major, M or N
// for mn-major) and o the other one, lives at
//   p + (c >> blk_shift) * blk_stride + o * ld + (c & (2^blk_shift - 1)),
// i.e. the contiguous index runs in blocks of 2^blk_shift elements (>= 8).
struct GemmOperand {
  const bf16* p;
  int64_t ld;          // stride of the other index, elements
  int blk_shift;       // log2 of the block length of the contiguous index
  int64_t blk_stride;  // distance between blocks, elements
  int kmajor;          // 1: K contiguous; 0: M (or N) contiguous
  int kvalid;          // M/N-contiguous operand: rows k >= kvalid (> 0) are read as row kvalid - 1,
                       // for a K padded to the 64-deep step (the other operand holds zeros there)
};

// C[m, n] at p + (n >> blk_shift) * blk_stride + m * ldc + (n & (2^blk_shift - 1)).
template <typename CT>
struct GemmOut {
  CT* p;
  int64_t ldc;
  int blk_shift;  // log2 of the block length of n (>= 3)
  int64_t blk_stride;
};

template <typename CT>
struct GemmParams {
  GemmOperand a, b;
  GemmOut<CT> c;
  int M, N, K;     // K a multiple of 64; M, N, block lengths multiples of 8
  int accumulate;  // fp32 C only: C += A B (else C = A B)
  int k_split;     // 0, or the K range (a multiple of 64) of each blockIdx.z: that range's
  float* partial;  // product goes to partial + z * M * N, fp32 [M][N], instead of C
};

__device__ __forceinline__ const bf16* gemm_elem(const GemmOperand& op, int64_t c, int64_t o) {
  return op.p + (c >> op.blk_shift) * op.blk_stride + o * op.ld + (c & ((int64_t(1) << op.blk_shift) - 1));
}

// Copy one operand's slice of a K tile into LDS. k-major: [128 mn][64 k]
// tile (row = mn); mn-major: [64 k][128 mn] tile (row = k). Indices past the
// matrix (ragged M or N) are clamped to its last row or chunk: those lanes'
// results are never stored.
template <int KMAJOR, int MODE>
__device__ __forceinline__ void gemm_load_tile(bf16* tile, const GemmOperand& op, int mn0, int MN, int k0, int wave,
                                               int lane) {
  if constexpr (KMAJOR) {
    constexpr int D = 64, CPR = D / 8, INSTR = 128 * CPR / 64;
#pragma unroll
    for (int i0 = 0; i0 < INSTR / 4; ++i0) {
      const int i = i0 * 4 + wave, slot = i * 64 + lane;
      const int r = slot / CPR, pos = slot % CPR, c = pos ^ swz<D, MODE>(r);
      const int mn = min(mn0 + r, MN - 1);
      __builtin_amdgcn_global_load_lds((const void*)gemm_elem(op, (int64_t)k0 + c * 8, mn), (lds_void*)(tile + i * 512),
                                       16, 0, 0);
    }
  } else {
    constexpr int D = 128, CPR = D / 8, INSTR = 64 * CPR / 64;
#pragma unroll
    for (int i0 = 0; i0 < INSTR / 4; ++i0) {
      const int i = i0 * 4 + wave, slot = i * 64 + lane;
      const int r = slot / CPR, pos = slot % CPR, c = pos ^ swz<D, MODE>(r);
      const int mn = min(mn0 + c * 8, MN - 8);
      __builtin_amdgcn_global_load_lds((const void*)gemm_elem(op, mn, min(k0 + r, op.kvalid - 1)),
                                       (lds_void*)(tile + i * 512), 16, 0, 0);
    }
  }
}

// Four 16-byte-per-lane global -> LDS copies from per-lane 64-bit addresses
// to LDS l, l + STEP, l + 2 STEP, l + 3 STEP (bytes; M0 saved and restored),
// issued from inline assembly so that the compiler does not track them: it
// then does not wait for them before LDS reads of the other buffer. They
// write no register; the caller waits for them by count (vmcnt) and a
// barrier before the destination is read.
template <unsigned STEP>
__device__ __forceinline__ void gemm_copy16x4_untracked(const void* a0, const void* a1, const void* a2, const void* a3,
                                                        lds_void* l) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)l);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_add_u32 m0, m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
      "s_add_u32 m0, m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, off\n\t"
      "s_add_u32 m0, m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, off\n\t"
      "s_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "s"(m0), "i"(STEP)
      : "memory", "scc");
}

// gemm_load_tile through the untracked copies: four copies per wave of a
// 4-wave group (wave = 0..3 within the group).
template <int KMAJOR, int MODE>
__device__ __forceinline__ void gemm_load_tile_untracked(bf16* tile, const GemmOperand& op, int mn0, int MN, int k0,
                                                         int wave, int lane) {
  const void* a[4];
#pragma unroll
  for (int i0 = 0; i0 < 4; ++i0) {
    const int i = i0 * 4 + wave, slot = i * 64 + lane;
    if constexpr (KMAJOR) {
      constexpr int D = 64, CPR = D / 8;
      const int r = slot / CPR, pos = slot % CPR, c = pos ^ swz<D, MODE>(r);
      a[i0] = gemm_elem(op, (int64_t)k0 + c * 8, min(mn0 + r, MN - 1));
    } else {
      constexpr int D = 128, CPR = D / 8;
      const int r = slot / CPR, pos = slot % CPR, c = pos ^ swz<D, MODE>(r);
      a[i0] = gemm_elem(op, min(mn0 + c * 8, MN - 8), min(k0 + r, op.kvalid - 1));
    }
  }
  gemm_copy16x4_untracked<4 * 1024>(a[0], a[1], a[2], a[3], (lds_void*)(tile + wave * 512));
}

// Operand fragment for MFMA step ks (k = 16 ks .. 16 ks + 15 of the tile) and
// the 32-row block mb of the operand's 128 M (or N) rows. NATURAL (both
// operands k-major): lane half h supplies k = 8h .. 8h + 7, one 16-byte read.
// Otherwise the k order of a P fragment (see the file comment): a transposed
// read for an mn-major tile, two 8-byte reads for a k-major one.
template <int KMAJOR, int NATURAL, int MODE>
__device__ __forceinline__ bf16x8 gemm_frag(const bf16* tile, int ks, int mb, int lane) {
  if constexpr (KMAJOR) {
    const int row = mb * 32 + (lane & 31), half = lane >> 5;
    if constexpr (NATURAL) return tile_row_frag<64, MODE>(tile, row, 2 * ks + half);
    const bf16* p0 = tile + tile_off<64, MODE>(row, 2 * ks) + 4 * half;
    const bf16* p1 = tile + tile_off<64, MODE>(row, 2 * ks + 1) + 4 * half;
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p0);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    return tile_tr_frag<128, MODE>(tile, 16 * ks, mb * 32, lane);
  }
}

// 4 waves, 128 x 128 tile of C per workgroup, each wave 64 x 64 (2 x 2 MFMA
// tiles of 32 x 32), K in steps of 64, LDS double-buffered (64 KiB). Each K
// step first reads all of its fragments from LDS into registers and only then
// issues the copies of the next K tile into the other buffer, so those copies
// fly while the MFMAs run (LDS reads issued after a copy would wait for it).
template <typename CT, int AK, int BK>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmParams<CT> p) {
  constexpr int MODE = kSwzAll;
  constexpr int NATURAL = AK && BK;
  __shared__ __attribute__((aligned(1024))) bf16 sA[2][128 * 64];
  __shared__ __attribute__((aligned(1024))) bf16 sB[2][128 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * 128, n0 = blockIdx.y * 128;
  const int wm = (wave & 1) * 2, wn = (wave >> 1) * 2;  // this wave's 32-row blocks of M and of N
  const int kb = p.k_split ? (int)blockIdx.z * p.k_split : 0;  // this workgroup's K range
  const int nk = (p.k_split ? min(p.k_split, p.K - kb) : p.K) / 64;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  gemm_load_tile<AK, MODE>(sA[0], p.a, m0, p.M, kb, wave, lane);
  gemm_load_tile<BK, MODE>(sB[0], p.b, n0, p.N, kb, wave, lane);
  wait_vm();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    bf16x8 af[4][2], bfr[4][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[ks][i] = gemm_frag<AK, NATURAL, MODE>(sA[cur], ks, wm + i, lane);
        bfr[ks][i] = gemm_frag<BK, NATURAL, MODE>(sB[cur], ks, wn + i, lane);
      }
    if (kt + 1 < nk) {
      gemm_load_tile<AK, MODE>(sA[cur ^ 1], p.a, m0, p.M, kb + (kt + 1) * 64, wave, lane);
      gemm_load_tile<BK, MODE>(sB[cur ^ 1], p.b, n0, p.N, kb + (kt + 1) * 64, wave, lane);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      // C^T tiles: lane = m (column of C^T), registers = n
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma32(acc[i][j], bfr[ks][j], af[ks][i]);
    wait_vm();
    __syncthreads();
  }

  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + (wm + i) * 32 + (lane & 31);
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + (wn + j) * 32 + 8 * g + 4 * half;  // registers 4g .. 4g+3: n .. n+3
        if (n >= p.N) continue;
        if (p.k_split) {
          floatx4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
          *reinterpret_cast<floatx4*>(p.partial + ((size_t)blockIdx.z * p.M + m) * p.N + n) = v;
          continue;
        }
        const int sh = min(p.c.blk_shift, 31);  // n < 2^31: a shift of 31 leaves block 0
        CT* dst = p.c.p + (int64_t)((unsigned)n >> sh) * p.c.blk_stride + (int64_t)m * p.c.ldc +
                  ((unsigned)n & ((1u << sh) - 1u));
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
        if constexpr (std::is_same<CT, float>::value) {
          if (p.accumulate) {
            const floatx4 old = *reinterpret_cast<const floatx4*>(dst);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = old[e] + v[e];
          }
          *reinterpret_cast<floatx4*>(dst) = v;
        } else {
          *reinterpret_cast<bf16x4*>(dst) = to_out4(v, bf16());
        }
      }
  }
}

// C (+)= the sum of n_split fp32 partial products [z][M][N], added in
// ascending z, written in C's layout (bf16: rounded once, at the end).
template <typename CT>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(const float* __restrict__ partial, int n_split, int M,
                                                                int N, GemmOut<CT> c, int accumulate) {
  const size_t n4 = (size_t)M * N / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(i * 4 / N), n = (int)(i * 4 % N);
    floatx4 v = *reinterpret_cast<const floatx4*>(partial + i * 4);
    for (int z = 1; z < n_split; ++z) v += *reinterpret_cast<const floatx4*>(partial + (size_t)z * M * N + i * 4);
    const int sh = min(c.blk_shift, 31);
    CT* dst = c.p + (int64_t)((unsigned)n >> sh) * c.blk_stride + (int64_t)m * c.ldc + ((unsigned)n & ((1u << sh) - 1u));
    if constexpr (std::is_same<CT, float>::value) {
      if (accumulate) v += *reinterpret_cast<const floatx4*>(dst);
      *reinterpret_cast<floatx4*>(dst) = v;
    } else {
      *reinterpret_cast<bf16x4*>(dst) = to_out4(v, bf16());
    }
  }
}

// The same product with a 256 x 256 C tile per workgroup of 8 waves (one
// workgroup per CU), each wave 128 x 64 (4 x 2 MFMA tiles), for problems with
// at least one such tile per CU. Each MFMA then reads 0.75 KiB of operands
// from LDS instead of 1 KiB, and each operand tile is copied once for twice
// the MFMAs. Operand tiles are two 128-row halves in the layout above (waves
// 0-3 copy one half, 4-7 the other), double-buffered (128 KiB of LDS).
template <typename CT, int AK, int BK>
__global__ __launch_bounds__(512, 1) void gemm_bf16_256_kernel(GemmParams<CT> p) {
  constexpr int MODE = kSwzAll;
  constexpr int NATURAL = AK && BK;
  __shared__ __attribute__((aligned(1024))) bf16 sA[2][2][128 * 64];
  __shared__ __attribute__((aligned(1024))) bf16 sB[2][2][128 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.x * 256, n0 = blockIdx.y * 256;
  const int wm = wave & 1;                         // this wave's 128-row half of M
  const int nh = wave >> 2, nb0 = (wave >> 1) & 1;  // its 128-column half of N, and 64-column quarter in it
  const int ch = wave >> 2, cw = wave & 3;         // the half this wave copies, its index among that half's 4 waves
  const int nk = p.K / 64;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  gemm_load_tile<AK, MODE>(sA[0][ch], p.a, m0 + 128 * ch, p.M, 0, cw, lane);
  gemm_load_tile<BK, MODE>(sB[0][ch], p.b, n0 + 128 * ch, p.N, 0, cw, lane);
  wait_vm();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // The next K tile's copies go out first, into the buffer the last step
    // read before its closing barrier; the untracked copies let this step's
    // fragment reads and MFMAs run while they fly.
    if (kt + 1 < nk) {
      gemm_load_tile_untracked<AK, MODE>(sA[cur ^ 1][ch], p.a, m0 + 128 * ch, p.M, (kt + 1) * 64, cw, lane);
      gemm_load_tile_untracked<BK, MODE>(sB[cur ^ 1][ch], p.b, n0 + 128 * ch, p.N, (kt + 1) * 64, cw, lane);
    }
    if constexpr (!AK && !BK) {
      // Both operands read transposed (two 8-byte reads per fragment): the
      // fragments of step ks + 1 are read while step ks's MFMAs run.
      bf16x8 af[2][4], bfr[2][2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[0][i] = gemm_frag<AK, NATURAL, MODE>(sA[cur][wm], 0, i, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[0][j] = gemm_frag<BK, NATURAL, MODE>(sB[cur][nh], 0, 2 * nb0 + j, lane);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c = ks & 1;
        if (ks + 1 < 4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) af[c ^ 1][i] = gemm_frag<AK, NATURAL, MODE>(sA[cur][wm], ks + 1, i, lane);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            bfr[c ^ 1][j] = gemm_frag<BK, NATURAL, MODE>(sB[cur][nh], ks + 1, 2 * nb0 + j, lane);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) mma32(acc[i][j], bfr[c][j], af[c][i]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 af[4], bfr[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = gemm_frag<AK, NATURAL, MODE>(sA[cur][wm], ks, i, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) bfr[j] = gemm_frag<BK, NATURAL, MODE>(sB[cur][nh], ks, 2 * nb0 + j, lane);
        // C^T tiles: lane = m (column of C^T), registers = n
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) mma32(acc[i][j], bfr[j], af[i]);
      }
    }
    wait_vm();
    __syncthreads();
  }

  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + i * 32 + (lane & 31);
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + nh * 128 + (2 * nb0 + j) * 32 + 8 * g + 4 * half;  // registers 4g .. 4g+3: n .. n+3
        if (n >= p.N) continue;
        const int sh = min(p.c.blk_shift, 31);
        CT* dst = p.c.p + (int64_t)((unsigned)n >> sh) * p.c.blk_stride + (int64_t)m * p.c.ldc +
                  ((unsigned)n & ((1u << sh) - 1u));
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
        if constexpr (std::is_same<CT, float>::value) {
          if (p.accumulate) {
            const floatx4 old = *reinterpret_cast<const floatx4*>(dst);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = old[e] + v[e];
          }
          *reinterpret_cast<floatx4*>(dst) = v;
        } else {
          *reinterpret_cast<bf16x4*>(dst) = to_out4(v, bf16());
        }
      }
  }
}

}  // namespace upipe
