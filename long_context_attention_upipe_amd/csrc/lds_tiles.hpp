// bf16 tiles in LDS for gfx950: row-major, XOR-swizzled 16-byte chunks,
// filled straight from global memory (global_load_lds_dwordx4, no register
// staging), read either as row fragments (ds_read_b128) or as transposed
// fragments (ds_read_b64_tr_b16), so one copy of a tile serves both MFMA
// operand orientations.
#pragma once

#include "common.hpp"

namespace upipe {

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef __attribute__((address_space(3))) void lds_void;

// Chunk c (16 bytes = 8 bf16) of row r lives at chunk position c ^ swz<D, M>(r).
// LDS has 64 four-byte banks (256 bytes per pass): a 16-byte-per-lane read is
// served 16 lanes at a time, an 8-byte-per-lane read 32 lanes at a time.
//  * Row-fragment reads (ds_read_b128): 16 lanes read one chunk of 16
//    consecutive rows; conflict-free when those 16 slots land on 16 different
//    16-byte bank groups.
//  * Transposed reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive chunks
//    (4-aligned) of an aligned group of 4 rows, then the same 4 rows + 8.
// Two layouts, chosen per kernel (each kernel fills and reads its own tiles):
//  * kSwzTr: transposed reads conflict-free, row reads 2-way; swz has period 8
//    in r, so the row+8 half of a transposed read is the first half's address
//    plus an immediate offset.
//  * kSwzAll: both read kinds conflict-free; swz has period 16, so the row+8
//    half needs an address of its own.
// d = 128 rows (256 bytes) span all banks; d = 64 rows (128 bytes) span half,
// the row's parity picking the half.
enum SwizzleMode { kSwzTr = 0, kSwzAll = 1 };

template <int D, int M>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "tiles are 64 or 128 elements wide");
  if constexpr (D == 128) {
    // low 2 bits of r pick the top 2 bits: distinct across each aligned group of 4 rows
    if constexpr (M == kSwzAll) return ((r & 3) << 2) | ((r >> 2) & 3);
    return ((r & 3) << 2) | ((r >> 2) & 1);
  } else {
    if constexpr (M == kSwzAll) {
      const int s = r >> 1;
      return ((s & 1) << 2) | ((s >> 1) & 3);
    }
    return ((r & 3) << 1) | ((r >> 2) & 1);
  }
}

// Element offset of chunk `chunk` of row `row` in a tile with D-element rows.
template <int D, int M = kSwzTr>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * D + ((chunk ^ swz<D, M>(row)) << 3);
}

// Row fragment: elements [8*chunk, 8*chunk + 8) of `row`.
template <int D, int M = kSwzTr>
__device__ __forceinline__ bf16x8 tile_row_frag(const bf16* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + tile_off<D, M>(row, chunk));
}

// Transposed fragment for an MFMA A/B operand whose contraction runs over the
// tile's rows: lane (m = lane & 31, half = lane >> 5) receives
//   X[rbase + c_row(e, half)][col0 + m],  e = 0..7,
// i.e. the 16 rows rbase..rbase+15 in the k-order of a P/dS fragment built
// from C registers 0..7 (or 8..15 with rbase + 16). Each of the two
// ds_read_b64_tr_b16 gathers 4 rows: within a 16-lane group, lane i gets
// element i & 3 of the 8-byte slot addressed by lane (i >> 2) + 4k as its
// k-th value, so lane j addresses row 4*half + (j >> 2), columns 4*(j & 3)..+3.
template <int D, int M = kSwzTr>
__device__ __forceinline__ bf16x8 tile_tr_frag(const bf16* tile, int rbase, int col0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int half = g >> 1, m0 = (g & 1) << 4;
  const int row = rbase + (half << 2) + (j >> 2);
  const int col = col0 + m0 + ((j & 3) << 2);
  const int chunk = col >> 3, sub = col & 7;
  const bf16* p0 = tile + row * D + ((chunk ^ swz<D, M>(row)) << 3) + sub;
  const bf16* p1 = tile + (row + 8) * D + ((chunk ^ swz<D, M>(row + 8)) << 3) + sub;
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p0);
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p1);
  const short8v c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Issue the copy of rows g_row0 .. g_row0 + ROWS - 1 of a [S][D] bf16 matrix
// into `tile` (rows past S - 1 repeat row S - 1: callers mask them). Each wave
// instruction fills 1 KiB of LDS, 16 bytes per lane, lane order; the lane
// picks the global chunk that belongs at its LDS position. Asynchronous:
// complete with wait_vm() and a barrier before reading.
template <int D, int ROWS, int NWAVES, int M = kSwzTr>
__device__ __forceinline__ void tile_load_async(bf16* tile, const bf16* g, int g_row0, int S, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int SLOTS = ROWS * CPR;
  constexpr int INSTR = SLOTS / 64;
  static_assert(SLOTS % 64 == 0, "tile must be a whole number of 1 KiB wave copies");
  static_assert(INSTR % NWAVES == 0, "wave copies must split evenly");
#pragma unroll
  for (int k = 0; k < INSTR / NWAVES; ++k) {
    const int i = k * NWAVES + wave;
    const int slot = i * 64 + lane;
    const int r = slot / CPR, pos = slot % CPR;
    const int c = pos ^ swz<D, M>(r);
    const int gr = min(g_row0 + r, S - 1);
    __builtin_amdgcn_global_load_lds((const void*)(g + (size_t)gr * D + c * 8), (lds_void*)(tile + i * 512), 16, 0,
                                     0);
  }
}

// Issue the copy of a ROWS x W block of a row-major bf16 matrix with row
// stride ld elements, starting at g, into `tile` (same LDS layout as
// tile_load_async with D = W). Every element must lie inside the matrix: the
// caller pads. Asynchronous, completed like tile_load_async.
template <int W, int ROWS, int NWAVES, int M = kSwzTr>
__device__ __forceinline__ void tile_load_rows_async(bf16* tile, const bf16* g, size_t ld, int wave, int lane) {
  constexpr int CPR = W / 8;
  constexpr int SLOTS = ROWS * CPR;
  constexpr int INSTR = SLOTS / 64;
  static_assert(SLOTS % 64 == 0, "tile must be a whole number of 1 KiB wave copies");
  static_assert(INSTR % NWAVES == 0, "wave copies must split evenly");
#pragma unroll
  for (int k = 0; k < INSTR / NWAVES; ++k) {
    const int i = k * NWAVES + wave;
    const int slot = i * 64 + lane;
    const int r = slot / CPR, pos = slot % CPR;
    const int c = pos ^ swz<W, M>(r);
    __builtin_amdgcn_global_load_lds((const void*)(g + (size_t)r * ld + c * 8), (lds_void*)(tile + i * 512), 16, 0,
                                     0);
  }
}

// Four of one wave's 16-byte-per-lane global -> LDS copies
// (global_load_lds_dwordx4 of base + the lane's offset o[k], base uniform),
// to LDS addresses l, l + step, l + 2 step, l + 3 step (bytes; the LDS address
// goes in M0, which is saved and restored), issued from inline assembly so
// that the compiler does not track them: it then neither waits for them
// before LDS reads of other buffers nor stops counting LDS reads in order
// while they are in flight. The caller orders them by hand: s_waitcnt vmcnt
// (they count like any vector load) and a barrier before the destination is
// read. Vector loads complete in issue order, so copies the compiler does
// not know of can only make its own vmcnt waits stricter, never too short.
template <unsigned STEP>
__device__ __forceinline__ void lds_copy16x4_untracked(const void* base, unsigned o0, unsigned o1, unsigned o2,
                                                       unsigned o3, lds_void* l) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)l);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %5\n\t"
      "s_add_u32 m0, m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %5\n\t"
      "s_add_u32 m0, m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %5\n\t"
      "s_add_u32 m0, m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %5\n\t"
      "s_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(base), "s"(m0), "i"(STEP)
      : "memory", "scc");
}

// The same with two copies (l, l + step).
template <unsigned STEP>
__device__ __forceinline__ void lds_copy16x2_untracked(const void* base, unsigned o0, unsigned o1, lds_void* l) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)l);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %3\n\t"
      "s_add_u32 m0, m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\t"
      "s_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "s"(base), "s"(m0), "i"(STEP)
      : "memory", "scc");
}

// The same with one copy.
__device__ __forceinline__ void lds_copy16x1_untracked(const void* base, unsigned o0, lds_void* l) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)l);
  unsigned saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_nop 0\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(o0), "s"(base), "s"(m0)
               : "memory");
}

// One 4-byte-per-lane copy from a per-lane 64-bit address, untracked like
// the above.
__device__ __forceinline__ void lds_copy4_untracked(const void* g, lds_void* l) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)l);
  unsigned saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_nop 0\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(g), "s"(m0)
               : "memory");
}

// tile_load_async / tile_load_rows_async through the untracked copies, for
// tiles that take one, two or four wave copies per wave.
template <int D, int ROWS, int NWAVES, int M = kSwzTr>
__device__ __forceinline__ void tile_load_untracked(bf16* tile, const bf16* g, int g_row0, int S, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int PER = ROWS * CPR / (64 * NWAVES);
  static_assert(ROWS * CPR == PER * 64 * NWAVES && (PER == 1 || PER == 2 || PER == 4), "1, 2 or 4 wave copies per wave");
  const bf16* base = g + (size_t)g_row0 * D;
  const int last = S - 1 - g_row0;  // rows past S - 1 repeat row S - 1
  unsigned o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int slot = (k * NWAVES + wave) * 64 + lane;
    const int r = slot / CPR, pos = slot % CPR;
    const int c = pos ^ swz<D, M>(r);
    o[k] = (unsigned)(min(r, last) * D + c * 8) * 2u;
  }
  if constexpr (PER == 4)
    lds_copy16x4_untracked<NWAVES * 1024>(base, o[0], o[1], o[2], o[3], (lds_void*)(tile + wave * 512));
  else if constexpr (PER == 2)
    lds_copy16x2_untracked<NWAVES * 1024>(base, o[0], o[1], (lds_void*)(tile + wave * 512));
  else
    lds_copy16x1_untracked(base, o[0], (lds_void*)(tile + wave * 512));
}
template <int W, int ROWS, int NWAVES, int M = kSwzTr>
__device__ __forceinline__ void tile_load_rows_untracked(bf16* tile, const bf16* g, int ld, int wave, int lane) {
  constexpr int CPR = W / 8;
  static_assert(ROWS * CPR == 4 * 64 * NWAVES, "four 1 KiB wave copies per wave");
  unsigned o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int slot = (k * NWAVES + wave) * 64 + lane;
    const int r = slot / CPR, pos = slot % CPR;
    const int c = pos ^ swz<W, M>(r);
    o[k] = (unsigned)(r * ld + c * 8) * 2u;
  }
  lds_copy16x4_untracked<NWAVES * 1024>(g, o[0], o[1], o[2], o[3], (lds_void*)(tile + wave * 512));
}

// Wait until at most N of this wave's vector loads (LDS copies included) are
// outstanding; they complete in issue order. N in {0, 4, 8}.
template <int N>
__device__ __forceinline__ void wait_vm_leave() {
  static_assert(N == 0 || N == 4 || N == 8, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Wait for this wave's outstanding global loads (including LDS copies).
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace upipe
