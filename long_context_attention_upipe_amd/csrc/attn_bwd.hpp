// Backward attention kernels for gfx950 (recompute-based).
//
// The probabilities are not stored by the forward; they are rebuilt from q, k
// and the saved lse, which is the attention-level form of the activation
// recomputation the talk relies on ("Road to 5 Million Tokens" talk summary,
// Chapters: activation checkpointing recomputes activations in the backward).
// With D_i = <dO_i, O_i>, P_ij = exp(s_ij - lse_i), dS_ij = P_ij (dP_ij - D_i):
//   dQ_i = tau sum_j dS_ij k_j,  dK_j = tau sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
//
// Two kernels keep every output owned by exactly one workgroup, so no
// floating-point atomics are needed and results are deterministic:
//  * attn_bwd_dkdv_kernel: kv-major. A workgroup owns 128 keys of one kv head
//    and walks the query heads of its group (ascending) and their query rows
//    i >= first key (ascending), accumulating dK^T and dV^T in registers.
//  * attn_bwd_dq_kernel: q-major. A workgroup owns 128 query rows of one head
//    and walks key tiles j <= i (ascending), accumulating dQ^T in registers.
#pragma once

#include "common.hpp"

namespace upipe {

template <typename T>
struct BwdParams {
  const T* q;          // pool: [hc][S][D]
  const T* k;          // pool: [nkv][S][D]
  const T* v;          // pool: [nkv][S][D]
  const T* dout;       // pool: [hc][S][D]
  const float* lse;    // caller lse rows of the chunk's first head, [hc][S]
  const float* negD;   // pool: -D = -<dO, O> per row, [hc][S]
  const float* lse2;   // pool: lse * log2(e) per row, [hc][S]
  T* dq;               // pool: [hc][S][D]
  float* dk_acc;       // pool: fp32 partial dK over earlier chunks, [nkv][S][D] (or null)
  float* dv_acc;
  T* dk_out;           // caller dk at the chunk's first kv head; row stride Hkv_total*D
  T* dv_out;
  int Hkv_total;
  int S;
  int hc;
  int heads_per_kv;
  int nkv;
  int n_qtiles;        // ceil(S / 128) (dQ kernel)
  int n_ktiles;        // ceil(S / 128) (dK/dV kernel)
  int causal;
  const int* doc_off;  // packed-document offsets o_0..o_n (device), or null
  int n_docs;          // n
  int acc_load;        // dK/dV start from dk_acc/dv_acc instead of zero
  int finalize;        // write tau*dK, dV as T to dk_out/dv_out (else fp32 to the acc)
  float scale;         // tau
  float scale_log2;    // tau * log2(e)
};

// ---------------------------------------------------------------------------
// dQ (q-major). S^T = K Q^T and dP^T = V dO^T put one query row per lane, so
// lse_i and D_i are per-lane scalars; dQ^T += K^T dS^T takes dS^T straight
// from registers with K stored transposed in LDS.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqShape {
  static constexpr int kThreads = 256;
  static constexpr int BQ = 128;
  static constexpr int BK = 64;
  static constexpr int EPV = 16 / sizeof(T);
  static constexpr int KLD = D + EPV;
  static constexpr int TLD = BK + EPV;
  static constexpr int NKS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int VPR = D / EPV;
  static constexpr int VPT = BK * VPR / kThreads;
  static constexpr int kLdsBytes = (2 * BK * KLD + D * TLD) * sizeof(T);
};

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(BwdParams<T> p) {
  typedef DqShape<T, D> Sh;
  typedef typename Frag<T>::type F;
  constexpr int BQ = Sh::BQ, BK = Sh::BK, EPV = Sh::EPV, KLD = Sh::KLD, TLD = Sh::TLD;
  constexpr int NKS = Sh::NKS, NDB = Sh::NDB, VPR = Sh::VPR, VPT = Sh::VPT;

  __shared__ __attribute__((aligned(16))) T sK[BK * KLD];
  __shared__ __attribute__((aligned(16))) T sV[BK * KLD];
  __shared__ __attribute__((aligned(16))) T sKT[D * TLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;

  const int t = blockIdx.x;
  const int qt = p.causal ? (p.n_qtiles - 1 - t / p.hc) : (t / p.hc);
  const int hl = t % p.hc;
  const int kvl = hl / p.heads_per_kv;
  const size_t head_elems = (size_t)S * D;
  const T* __restrict__ Q = p.q + (size_t)hl * head_elems;
  const T* __restrict__ dO = p.dout + (size_t)hl * head_elems;
  const T* __restrict__ K = p.k + (size_t)kvl * head_elems;
  const T* __restrict__ V = p.v + (size_t)kvl * head_elems;

  const int row0 = qt * BQ;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + col;
  const bool row_ok = my_row < S;

  F qf[NKS], df[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = row_ok ? load_frag(Q + (size_t)my_row * D + ks * 16 + half * 8) : F{};
    df[ks] = row_ok ? load_frag(dO + (size_t)my_row * D + ks * 16 + half * 8) : F{};
  }
  const float lse2 = row_ok ? p.lse[(size_t)hl * S + my_row] * kLog2e : 0.f;
  const float nD = row_ok ? p.negD[(size_t)hl * S + my_row] : 0.f;

  // Key windows as in the forward kernel.
  const int last_row = min(S, row0 + BQ) - 1;
  const DocSpan kw = key_window(p.doc_off, p.n_docs, min(my_row, S - 1), S, p.causal);
  const int w_first_min = __builtin_amdgcn_readlane(kw.first, 0);
  const int w_first_max = __builtin_amdgcn_readlane(kw.first, 31);
  const int w_last_min = __builtin_amdgcn_readlane(kw.last, 0);
  const int w_last_max = __builtin_amdgcn_readlane(kw.last, 31);
  const int kt_begin = p.doc_off ? key_window(p.doc_off, p.n_docs, row0, S, p.causal).first / BK : 0;
  const int kt_end = key_window(p.doc_off, p.n_docs, last_row, S, p.causal).last / BK + 1;

  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};

  uint4 kreg[VPT], vreg[VPT];
  auto load_tile = [&](int kt) {
    const int key0 = kt * BK;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * Sh::kThreads;
      // key-fastest: the transposed K stores of a wave hit consecutive addresses
      const int r = idx % BK, c = idx / BK;
      const bool ok = key0 + r < S;
      kreg[i] = ok ? *reinterpret_cast<const uint4*>(K + (size_t)(key0 + r) * D + c * EPV) : uint4{0, 0, 0, 0};
      vreg[i] = ok ? *reinterpret_cast<const uint4*>(V + (size_t)(key0 + r) * D + c * EPV) : uint4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * Sh::kThreads;
      const int r = idx % BK, c = idx / BK;
      *reinterpret_cast<uint4*>(sK + r * KLD + c * EPV) = kreg[i];
      *reinterpret_cast<uint4*>(sV + r * KLD + c * EPV) = vreg[i];
      const int pos = perm16(r);
      const T* ke = reinterpret_cast<const T*>(&kreg[i]);
#pragma unroll
      for (int e = 0; e < EPV; ++e) sKT[(c * EPV + e) * TLD + pos] = ke[e];
    }
  };

  load_tile(kt_begin);
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < kt_end) load_tile(kt + 1);

    const int key0 = kt * BK;
    const bool active = (wrow0 < S) && key0 + BK - 1 >= w_first_min && key0 <= w_last_max;
    if (!active) continue;

    floatx16 s[2], dp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = floatx16{};
      dp[b] = floatx16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const F kf = load_frag(sK + (b * 32 + col) * KLD + ks * 16 + half * 8);
        mma32(s[b], kf, qf[ks]);
        const F vf = load_frag(sV + (b * 32 + col) * KLD + ks * 16 + half * 8);
        mma32(dp[b], vf, df[ks]);
      }
    }

    const bool need_mask = key0 < w_first_max || key0 + BK - 1 > w_last_min;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float pij = __builtin_amdgcn_exp2f(fmaf(s[b][j], p.scale_log2, -lse2));
        if (need_mask) {
          const int key = key0 + b * 32 + c_row(j, half);
          if (key < kw.first || key > kw.last) pij = 0.f;
        }
        s[b][j] = pij * (dp[b][j] + nD);  // dS^T
      }

#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 dv8;
#pragma unroll
        for (int e = 0; e < 8; ++e) dv8[e] = s[b][st * 8 + e];
        const F dsf = to_frag(dv8, T());
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const F ktf = load_frag(sKT + (db * 32 + col) * TLD + b * 32 + st * 16 + half * 8);
          mma32(acc[db], ktf, dsf);
        }
      }
  }

  if (row_ok) {
    T* dQ = p.dq + (size_t)hl * head_elems + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[db][jg * 4 + e] * p.scale;
        *reinterpret_cast<typename Vec4<T>::type*>(dQ + db * 32 + jg * 8 + half * 4) = to_out4(v4, T());
      }
  }
}

// ---------------------------------------------------------------------------
// dK / dV (kv-major). S = Q K^T and dP = dO V^T put one key per lane (column);
// dV^T += dO^T P and dK^T += Q^T dS take P and dS straight from registers,
// with Q and dO stored both row-major and transposed in LDS.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkvShape {
  static constexpr int kThreads = 256;
  static constexpr int BKV = 128;           // keys per workgroup (32 per wave)
  static constexpr int BQ = 32;             // query rows per inner step
  static constexpr int EPV = 16 / sizeof(T);
  static constexpr int RLD = D + EPV;       // row-major tile stride
  static constexpr int TLD = BQ + EPV;      // transposed tile stride
  static constexpr int NKS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int VPR = D / EPV;
  static constexpr int VPT = BQ * VPR / kThreads;  // vectors per thread per tensor
  static constexpr int kLdsBytes = 2 * (BQ * RLD + D * TLD) * sizeof(T) + 2 * BQ * 4;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(BwdParams<T> p) {
  typedef DkvShape<T, D> Sh;
  typedef typename Frag<T>::type F;
  constexpr int BKV = Sh::BKV, BQ = Sh::BQ, EPV = Sh::EPV, RLD = Sh::RLD, TLD = Sh::TLD;
  constexpr int NKS = Sh::NKS, NDB = Sh::NDB, VPR = Sh::VPR, VPT = Sh::VPT;
  static_assert(VPT >= 1 && VPT * Sh::kThreads == BQ * VPR, "q block must split evenly over threads");

  __shared__ __attribute__((aligned(16))) T sQ[BQ * RLD];
  __shared__ __attribute__((aligned(16))) T sQT[D * TLD];
  __shared__ __attribute__((aligned(16))) T sO[BQ * RLD];   // dO rows
  __shared__ __attribute__((aligned(16))) T sOT[D * TLD];   // dO transposed
  __shared__ __attribute__((aligned(16))) float sL[BQ];     // lse * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[BQ];     // -D

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;

  // kv tile 0 has the most query rows under a causal mask: heaviest first.
  const int t = blockIdx.x;
  const int kt = t / p.nkv;
  const int g = t % p.nkv;
  const size_t head_elems = (size_t)S * D;
  const T* __restrict__ K = p.k + (size_t)g * head_elems;
  const T* __restrict__ V = p.v + (size_t)g * head_elems;

  const int key0 = kt * BKV;
  const int wkey0 = key0 + wave * 32;
  const int my_key = wkey0 + col;
  const bool key_ok = my_key < S;

  // K^T and V^T operands (B of S = Q K^T and dP = dO V^T): lane holds row my_key.
  F kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = key_ok ? load_frag(K + (size_t)my_key * D + ks * 16 + half * 8) : F{};
    vf[ks] = key_ok ? load_frag(V + (size_t)my_key * D + ks * 16 + half * 8) : F{};
  }

  floatx16 dk[NDB], dv[NDB];
  if (p.acc_load) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 a = key_ok ? *reinterpret_cast<const floatx4*>(p.dk_acc + (size_t)g * head_elems + (size_t)my_key * D +
                                                                db * 32 + jg * 8 + half * 4)
                           : floatx4{};
        floatx4 b = key_ok ? *reinterpret_cast<const floatx4*>(p.dv_acc + (size_t)g * head_elems + (size_t)my_key * D +
                                                                db * 32 + jg * 8 + half * 4)
                           : floatx4{};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[db][jg * 4 + e] = a[e];
          dv[db][jg * 4 + e] = b[e];
        }
      }
  } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dk[db] = floatx16{};
      dv[db] = floatx16{};
    }
  }

  // Query rows that attend to this lane's key, [rw.first, rw.last]; both
  // bounds grow with the key, so lanes 0 and 31 give the wave's extremes and
  // the workgroup's first and last keys its row-block range [qb0, qb_top].
  const int last_key = min(S, key0 + BKV) - 1;
  DocSpan rw = row_window(p.doc_off, p.n_docs, min(my_key, S - 1), S, p.causal);
  if (p.causal) rw.first = my_key;  // a key past the end has no rows
  const int w_first_min = __builtin_amdgcn_readlane(rw.first, 0);
  const int w_first_max = __builtin_amdgcn_readlane(rw.first, 31);
  const int w_last_min = __builtin_amdgcn_readlane(rw.last, 0);
  const int w_last_max = __builtin_amdgcn_readlane(rw.last, 31);
  const int qb0 = row_window(p.doc_off, p.n_docs, key0, S, p.causal).first / BQ;
  const int qb_top = row_window(p.doc_off, p.n_docs, last_key, S, p.causal).last / BQ;
  const int steps_per_head = qb_top - qb0 + 1;
  const int n_steps = p.heads_per_kv * steps_per_head;

  uint4 qreg[VPT], oreg[VPT];
  float lreg = 0.f, dreg = 0.f;
  auto load_block = [&](int step) {
    const int hi = step / steps_per_head;
    const int qb = qb0 + step % steps_per_head;
    const int hl = g * p.heads_per_kv + hi;
    const T* Q = p.q + (size_t)hl * head_elems;
    const T* dO = p.dout + (size_t)hl * head_elems;
    const int r0 = qb * BQ;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * Sh::kThreads;
      const int r = idx % BQ, c = idx / BQ;  // row-fastest for the transposed stores
      const bool ok = r0 + r < S;
      qreg[i] = ok ? *reinterpret_cast<const uint4*>(Q + (size_t)(r0 + r) * D + c * EPV) : uint4{0, 0, 0, 0};
      oreg[i] = ok ? *reinterpret_cast<const uint4*>(dO + (size_t)(r0 + r) * D + c * EPV) : uint4{0, 0, 0, 0};
    }
    if (tid < BQ) {
      const bool ok = r0 + tid < S;
      lreg = ok ? p.lse[(size_t)hl * S + r0 + tid] * kLog2e : 0.f;
      dreg = ok ? p.negD[(size_t)hl * S + r0 + tid] : 0.f;
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int idx = tid + i * Sh::kThreads;
      const int r = idx % BQ, c = idx / BQ;
      *reinterpret_cast<uint4*>(sQ + r * RLD + c * EPV) = qreg[i];
      *reinterpret_cast<uint4*>(sO + r * RLD + c * EPV) = oreg[i];
      const int pos = perm16(r);
      const T* qe = reinterpret_cast<const T*>(&qreg[i]);
      const T* oe = reinterpret_cast<const T*>(&oreg[i]);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        sQT[(c * EPV + e) * TLD + pos] = qe[e];
        sOT[(c * EPV + e) * TLD + pos] = oe[e];
      }
    }
    if (tid < BQ) {
      sL[tid] = lreg;
      sD[tid] = dreg;
    }
  };

  if (n_steps > 0) load_block(0);
  for (int step = 0; step < n_steps; ++step) {
    const int qb = qb0 + step % steps_per_head;
    __syncthreads();
    store_block();
    __syncthreads();
    if (step + 1 < n_steps) load_block(step + 1);

    const int r0 = qb * BQ;
    const bool active = (wkey0 < S) && r0 + BQ - 1 >= w_first_min && r0 <= w_last_max;
    if (!active) continue;

    floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const F qa = load_frag(sQ + col * RLD + ks * 16 + half * 8);
      mma32(s, qa, kf[ks]);
      const F oa = load_frag(sO + col * RLD + ks * 16 + half * 8);
      mma32(dp, oa, vf[ks]);
    }

    const bool need_mask = r0 < w_first_max || r0 + BQ - 1 > w_last_min;
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const floatx4 l4 = *reinterpret_cast<const floatx4*>(sL + jg * 8 + half * 4);
      const floatx4 d4 = *reinterpret_cast<const floatx4*>(sD + jg * 8 + half * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = jg * 4 + e;
        float pij = __builtin_amdgcn_exp2f(fmaf(s[j], p.scale_log2, -l4[e]));
        if (need_mask) {
          const int row = r0 + c_row(j, half);
          if (row < rw.first || row > rw.last) pij = 0.f;
        }
        s[j] = pij;                     // P
        dp[j] = pij * (dp[j] + d4[e]);  // dS
      }
    }

#pragma unroll
    for (int st = 0; st < 2; ++st) {
      floatx8 p8, d8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p8[e] = s[st * 8 + e];
        d8[e] = dp[st * 8 + e];
      }
      const F pf = to_frag(p8, T());
      const F dsf = to_frag(d8, T());
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const F oa = load_frag(sOT + (db * 32 + col) * TLD + st * 16 + half * 8);
        mma32(dv[db], oa, pf);
        const F qa = load_frag(sQT + (db * 32 + col) * TLD + st * 16 + half * 8);
        mma32(dk[db], qa, dsf);
      }
    }
  }

  if (!key_ok) return;
  if (p.finalize) {
    T* dK = p.dk_out + ((size_t)my_key * p.Hkv_total + g) * D;
    T* dV = p.dv_out + ((size_t)my_key * p.Hkv_total + g) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dk[db][jg * 4 + e] * p.scale;
          b[e] = dv[db][jg * 4 + e];
        }
        *reinterpret_cast<typename Vec4<T>::type*>(dK + db * 32 + jg * 8 + half * 4) = to_out4(a, T());
        *reinterpret_cast<typename Vec4<T>::type*>(dV + db * 32 + jg * 8 + half * 4) = to_out4(b, T());
      }
  } else {
    float* aK = p.dk_acc + (size_t)g * head_elems + (size_t)my_key * D;
    float* aV = p.dv_acc + (size_t)g * head_elems + (size_t)my_key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dk[db][jg * 4 + e];
          b[e] = dv[db][jg * 4 + e];
        }
        *reinterpret_cast<floatx4*>(aK + db * 32 + jg * 8 + half * 4) = a;
        *reinterpret_cast<floatx4*>(aV + db * 32 + jg * 8 + half * 4) = b;
      }
  }
}

}  // namespace upipe
