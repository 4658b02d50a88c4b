// Forward attention kernel for gfx950.
//
// Computes, for each query row i of each head of a chunk, the exact softmax
// attention over keys j <= i (all keys if non-causal) with an online softmax
// over key tiles, and saves lse = ln sum_j exp(s_ij)
// ("Road to 5 Million Tokens" talk summary, Chapters: under Ulysses each GPU
// runs attention over the whole sequence for its heads; MaxText long-context
// article: causal look-back over all earlier positions).
//
// Work decomposition. One workgroup (4 waves) owns 128 query rows of one
// head; each wave owns 32 rows. Keys are visited in tiles of 64 in ascending
// order, every tile staged once in LDS and shared by the 4 waves.
//
// Orientation. Scores are formed transposed, S^T = K Q^T (32 keys x 32 rows per
// MFMA tile), so every lane owns one query row (column) and 16 of its scores;
// the other 16 live in lane^32. Row max / row sum therefore need a single
// cross-half exchange per tile, and the running max, sum and rescale factor
// are per-lane scalars. The output is accumulated transposed too,
// O^T += V^T P^T, whose B operand (P^T) is taken straight from the score
// registers; V is stored transposed in LDS, in the matching key order.
#pragma once

#include "common.hpp"

namespace upipe {

template <typename T>
struct FwdParams {
  const T* q;        // pool: chunk q rows, [hc][S][D]
  const T* k;        // pool: chunk kv heads, [nkv][S][D]
  const T* v;        // pool: fp32 [nkv][S][D]; bf16 transposed, [nkv][Sp/64][D][64] (pack_vt_kernel)
  int Sp;            // bf16: S rounded up to 64
  T* o;              // pool: chunk output rows, [hc][S][D]
  T* o_lo;           // caller out_lo at the chunk's first head (row stride H*D), or null
  int H;             // caller heads per row (out_lo row stride in heads)
  float* lse;        // caller lse rows of the chunk's first head, [hc][S]
  int S;
  int hc;            // heads in the chunk
  int heads_per_kv;  // chunk head hl reads pool kv head hl / heads_per_kv
  int n_qtiles;      // ceil(S / 128)
  int causal;
  const int* doc_off;  // packed-document offsets o_0..o_n (device), or null
  int n_docs;          // n
  float scale_log2;  // tau * log2(e)
};

template <typename T, int D>
struct FwdShape {
  static constexpr int kThreads = 256;
  static constexpr int BQ = 128;            // query rows per workgroup
  static constexpr int BK = 64;             // keys per tile
  static constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
  static constexpr int KLD = D + EPV;       // K tile row stride (elements)
  static constexpr int VLD = BK + EPV;      // V^T tile row stride (elements)
  static constexpr int NKS = D / 16;        // 16-deep contraction steps over d
  static constexpr int NDB = D / 32;        // 32-row blocks of d
  static constexpr int VPR = D / EPV;       // 16-byte vectors per K/V row
  static constexpr int VPT = BK * VPR / kThreads;  // vectors per thread per tile
  static constexpr int kLdsBytes = (BK * KLD + D * VLD) * sizeof(T);
};

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_kernel(FwdParams<T> p) {
  typedef FwdShape<T, D> Sh;
  typedef typename Frag<T>::type F;
  constexpr int BQ = Sh::BQ, BK = Sh::BK, EPV = Sh::EPV, KLD = Sh::KLD, VLD = Sh::VLD;
  constexpr int NKS = Sh::NKS, NDB = Sh::NDB, VPR = Sh::VPR, VPT = Sh::VPT;
  static_assert(VPT * Sh::kThreads == BK * VPR, "tile must split evenly over threads");

  __shared__ __attribute__((aligned(16))) T sK[BK * KLD];
  __shared__ __attribute__((aligned(16))) T sVT[D * VLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;

  // Heaviest query tiles first: under a causal mask tile qt costs ~ qt + 1
  // key tiles, so the long ones start early and the short ones fill the tail.
  const int t = blockIdx.x;
  const int qt = p.causal ? (p.n_qtiles - 1 - t / p.hc) : (t / p.hc);
  const int hl = t % p.hc;
  const int kvl = hl / p.heads_per_kv;
  const size_t head_elems = (size_t)S * D;
  const T* __restrict__ Q = p.q + (size_t)hl * head_elems;
  const T* __restrict__ K = p.k + (size_t)kvl * head_elems;
  const T* __restrict__ V = p.v + (size_t)kvl * head_elems;

  const int row0 = qt * BQ;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + col;

  // Q^T operand (B of S^T = K Q^T): lane holds Q[my_row][16ks + 8half + 0..7].
  F qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (my_row < S)
      qf[ks] = load_frag(Q + (size_t)my_row * D + ks * 16 + half * 8);
    else
      qf[ks] = F{};
  }

  // Keys this lane's row attends to, [kw.first, kw.last]; both bounds grow
  // with the row, so lanes 0 and 31 give the wave's extremes and the
  // workgroup's first and last rows its key-tile range.
  const int last_row = min(S, row0 + BQ) - 1;
  const DocSpan kw = key_window(p.doc_off, p.n_docs, min(my_row, S - 1), S, p.causal);
  const int w_first_min = __builtin_amdgcn_readlane(kw.first, 0);
  const int w_first_max = __builtin_amdgcn_readlane(kw.first, 31);
  const int w_last_min = __builtin_amdgcn_readlane(kw.last, 0);
  const int w_last_max = __builtin_amdgcn_readlane(kw.last, 31);
  const int kt_begin = p.doc_off ? key_window(p.doc_off, p.n_docs, row0, S, p.causal).first / BK : 0;
  const int kt_end = key_window(p.doc_off, p.n_docs, last_row, S, p.causal).last / BK + 1;

  floatx16 o_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o_acc[db] = floatx16{};
  const float NEG_INF = -__builtin_inff();
  float m_run = NEG_INF;  // running max of s * tau * log2(e)
  float l_run = 0.f;      // this lane's half of the running sum

  // Register staging of the next K/V tile. K vectors are taken row by row
  // (coalesced); V vectors key-fastest so that the transposed LDS stores of a
  // wave fall on consecutive addresses.
  uint4 kreg[VPT], vreg[VPT];
  auto load_tile = [&](int kt) {
    const int key0 = kt * BK;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * Sh::kThreads;
      const int kr = idx / VPR, kc = idx % VPR;
      const int vr = idx % BK, vc = idx / BK;
      kreg[i] = (key0 + kr < S) ? *reinterpret_cast<const uint4*>(K + (size_t)(key0 + kr) * D + kc * EPV)
                                : uint4{0, 0, 0, 0};
      vreg[i] = (key0 + vr < S) ? *reinterpret_cast<const uint4*>(V + (size_t)(key0 + vr) * D + vc * EPV)
                                : uint4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * Sh::kThreads;
      const int kr = idx / VPR, kc = idx % VPR;
      *reinterpret_cast<uint4*>(sK + kr * KLD + kc * EPV) = kreg[i];
      const int vr = idx % BK, vc = idx / BK;
      const int pos = perm16(vr);
      const T* ve = reinterpret_cast<const T*>(&vreg[i]);
#pragma unroll
      for (int e = 0; e < EPV; ++e) sVT[(vc * EPV + e) * VLD + pos] = ve[e];
    }
  };

  load_tile(kt_begin);
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    __syncthreads();
    if (kt + 1 < kt_end) load_tile(kt + 1);  // in flight while this tile computes

    const int key0 = kt * BK;
    const bool active = (wrow0 < S) && key0 + BK - 1 >= w_first_min && key0 <= w_last_max;
    if (!active) continue;

    // S^T = K Q^T: two 32-key blocks.
    floatx16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = floatx16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const F kf = load_frag(sK + (b * 32 + col) * KLD + ks * 16 + half * 8);
        mma32(s[b], kf, qf[ks]);
      }
    }

    const bool need_mask = key0 < w_first_max || key0 + BK - 1 > w_last_min;
    if (need_mask) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = key0 + b * 32 + c_row(j, half);
          if (key < kw.first || key > kw.last) s[b][j] = NEG_INF;
        }
    }

    float mx = NEG_INF;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[b][j]);
    mx = wave_xor32_max(mx);
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[b][j] = __builtin_amdgcn_exp2f(fmaf(s[b][j], p.scale_log2, -m_use));
        psum += s[b][j];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o_acc[db] *= alpha;

    // O^T += V^T P^T, 16 keys per step.
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 pv;
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = s[b][st * 8 + e];
        const F pf = to_frag(pv, T());
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const F vf = load_frag(sVT + (db * 32 + col) * VLD + b * 32 + st * 16 + half * 8);
          mma32(o_acc[db], vf, pf);
        }
      }
  }

  const float l_tot = wave_xor32_sum(l_run);
  if (my_row < S) {
    const float inv = 1.f / l_tot;
    T* O = p.o + (size_t)hl * head_elems + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = o_acc[db][jg * 4 + e] * inv;
        *reinterpret_cast<typename Vec4<T>::type*>(O + db * 32 + jg * 8 + half * 4) = to_out4(o4, T());
      }
    if (half == 0) p.lse[(size_t)hl * S + my_row] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace upipe
