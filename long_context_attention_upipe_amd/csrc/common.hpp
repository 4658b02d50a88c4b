// Shared device-side building blocks for the gfx950 attention kernels:
// element types, 8-element MFMA operand fragments and the 32x32 MFMA step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace upipe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One MFMA operand fragment: the 8 consecutive contraction elements a lane
// supplies for a 16-deep step of a 32x32 output tile. For bf16 this is the
// operand of one v_mfma_f32_32x32x16_bf16; for fp32 it feeds eight
// v_mfma_f32_32x32x2_f32 (element e of every lane in the e-th one), so the
// contraction pairs the same (lane half, element) slots of A and B either way.
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef floatx8 type; };

__device__ __forceinline__ void mma32(floatx16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void mma32(floatx16& c, const floatx8& a, const floatx8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
}

// Load one fragment (8 consecutive elements, 16-byte aligned).
__device__ __forceinline__ bf16x8 load_frag(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ floatx8 load_frag(const float* p) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
  const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round 8 fp32 values to an operand fragment (bf16: round to nearest even).
__device__ __forceinline__ bf16x8 to_frag(const floatx8& x, bf16) {
  return __builtin_convertvector(x, bf16x8);
}
__device__ __forceinline__ floatx8 to_frag(const floatx8& x, float) { return x; }

// Element-wise fp32 -> T for output stores.
__device__ __forceinline__ bf16x4 to_out4(const floatx4& x, bf16) {
  return __builtin_convertvector(x, bf16x4);
}
__device__ __forceinline__ floatx4 to_out4(const floatx4& x, float) { return x; }

template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef floatx4 type; };

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// C/D layout of a 32x32 MFMA tile: lane l owns column (l & 31); its register
// j holds row ((j >> 2) << 3) + ((l >> 5) << 2) + (j & 3).
__device__ __forceinline__ int c_row(int j, int half) { return ((j >> 2) << 3) + (half << 2) + (j & 3); }

// The k-order of a P/dS operand built straight from C registers 8s..8s+7 of a
// 32-row tile: slot (half, e) of step s holds tile row c_row(8s + e, half).
// Operands read from LDS use the same order, so rows of a 16-row group are
// stored at position perm16(row) = row with bits 2 and 3 swapped.
__host__ __device__ __forceinline__ int perm16(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Combine a value with the one held by lane ^ 32, without going through LDS:
// v_permlane32_swap of x with itself returns {x[0..31], x[0..31]} and
// {x[32..63], x[32..63]}, so every lane sees its own value and its partner's.
__device__ __forceinline__ float wave_xor32_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_xor32_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Packed documents (MaxText article on long-context training, the note that
// several samples packed into one sequence need no padding): offsets
// o_0 = 0 <= o_1 <= ... <= o_n = S in device memory; document m holds
// positions o_m .. o_{m+1} - 1 and a position attends only within its own
// document. doc_span(i) returns the first and last position of the document
// holding position i (0 <= i < S) by binary search. It reads only o_0 .. o_n,
// and its results are clamped to [0, i] and [i, S - 1], so offsets that break
// the rules give wrong numbers but never an access outside the sequence.
struct DocSpan {
  int first, last;
};
__device__ __forceinline__ DocSpan doc_span(const int* __restrict__ off, int n, int i, int S) {
  int lo = 0, hi = n;  // o_lo <= i < o_hi for well-formed offsets
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= i)
      lo = mid;
    else
      hi = mid;
  }
  return {min(max(off[lo], 0), i), max(min(off[lo + 1] - 1, S - 1), i)};
}

// Keys that query row i attends to, [first, last]: up to the row itself when
// causal, and inside the row's document when off is set.
__device__ __forceinline__ DocSpan key_window(const int* __restrict__ off, int n, int i, int S, int causal) {
  DocSpan w = {0, causal ? i : S - 1};
  if (off) {
    const DocSpan d = doc_span(off, n, i, S);
    w.first = d.first;
    if (!causal) w.last = d.last;
  }
  return w;
}

// Query rows that attend to key j, [first, last]: from the key itself when
// causal, and inside the key's document when off is set.
__device__ __forceinline__ DocSpan row_window(const int* __restrict__ off, int n, int j, int S, int causal) {
  DocSpan w = {causal ? j : 0, S - 1};
  if (off) {
    const DocSpan d = doc_span(off, n, j, S);
    if (!causal) w.first = d.first;
    w.last = d.last;
  }
  return w;
}

}  // namespace upipe
