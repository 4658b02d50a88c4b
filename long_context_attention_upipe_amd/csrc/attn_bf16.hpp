// bf16 attention kernels for gfx950: forward, dQ and dK/dV.
//
// Same mathematics, orientation and determinism contract as the generic
// kernels (attn_fwd.hpp, attn_bwd.hpp), re-tiled for bf16 on CDNA4:
//  * K/V (forward, dQ) and Q/dO (dK/dV) tiles go global -> LDS directly, into
//    double-buffered XOR-swizzled row-major tiles (lds_tiles.hpp): one barrier
//    per tile, no staging registers;
//  * operands that contract over a tile's rows (K^T in dS K, dO^T in dV, Q^T
//    in dK) are read transposed from the same row-major tile with
//    ds_read_b64_tr_b16 instead of keeping a second, transposed copy; the
//    forward, whose only use of V is V^T, gets V transposed in the pool
//    instead, so all of its reads are ds_read_b128 (twice the bytes per LDS
//    instruction of the transposed read);
//  * register budgets fit two waves per SIMD, so one wave's softmax VALU
//    work overlaps the other wave's MFMAs.
#pragma once

#include "attn_bwd.hpp"
#include "attn_fwd.hpp"
#include "lds_tiles.hpp"

namespace upipe {

// Tile sizes of the bf16 kernels. The host sizes their grids from these same
// constants (one workgroup per kFwdRows query rows, per kDqRows rows, per
// kDkvKeys keys of each head), so a kernel and its launch cannot disagree.
struct Bf16Tiles {
  static constexpr int kFwdRows = 128, kFwdKeys = 64;  // forward: rows per workgroup, keys per tile
  static constexpr int kFwdPpRows = 256;               // the two-group forward's rows per workgroup
  static constexpr int kDqRows = 128, kDqKeys = 64;    // dQ: rows per workgroup, keys per tile
  static constexpr int kDqPpRows = 256, kDqPpKeys = 32;  // the two-group dQ: rows per workgroup, keys per tile
  static constexpr int kDkvKeys = 128, kDkvRows = 32;  // dK/dV: keys per workgroup, rows per step
};

// ---------------------------------------------------------------------------
// Forward: 4 waves x 32 query rows, 64-key tiles.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(FwdParams<bf16> p) {
  constexpr int BQ = Bf16Tiles::kFwdRows, BK = Bf16Tiles::kFwdKeys, NKS = D / 16, NDB = D / 32;
  static_assert(BQ == 4 * 32 && BK == 64, "4 waves x 32 rows; two 32-key blocks per tile");
  // K tiles [BK keys][D]; V tiles transposed, [D][BK positions] (pack_vt_kernel
  // blocks, one contiguous block per tile), so both operands are read as
  // 16-byte row fragments. Both layouts
  // are conflict-free for row reads (kSwzAll).
  __shared__ __attribute__((aligned(1024))) bf16 sK[2][BK * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV[2][BK * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;

  // Workgroups go to the 8 XCDs round-robin (index mod 8). Inside each
  // full block of 64 indices, XCD x takes the 8 consecutive tiles 8x .. 8x+7
  // of the block, so the workgroups that share one L2 stream the same K/V
  // tiles; the order across blocks stays heaviest first.
  const int t0 = blockIdx.x;
  const int t = (t0 / 64 + 1) * 64 <= (int)gridDim.x ? (t0 & ~63) | ((t0 & 7) << 3) | ((t0 >> 3) & 7) : t0;
  const int qt = p.causal ? (p.n_qtiles - 1 - t / p.hc) : (t / p.hc);
  const int hl = t % p.hc;
  const int kvl = hl / p.heads_per_kv;
  const size_t head_elems = (size_t)S * D;
  const bf16* __restrict__ Q = p.q + (size_t)hl * head_elems;
  const bf16* __restrict__ K = p.k + (size_t)kvl * head_elems;
  const bf16* __restrict__ VT = p.v + (size_t)kvl * D * p.Sp;

  const int row0 = qt * BQ;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + col;

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

  tile_load_async<D, BK, 4, kSwzAll>(sK[kt_begin & 1], K, kt_begin * BK, S, wave, lane);
  tile_load_rows_async<BK, D, 4, kSwzAll>(sV[kt_begin & 1], VT + (size_t)kt_begin * BK * D, BK, wave, lane);

  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = my_row < S ? *reinterpret_cast<const bf16x8*>(Q + (size_t)my_row * D + ks * 16 + half * 8) : bf16x8{};

  floatx16 o_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o_acc[db] = floatx16{};
  const float NEG_INF = -__builtin_inff();
  float m_run = NEG_INF;
  float l_run = 0.f;

  wait_vm();
  __syncthreads();
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < kt_end) {
      tile_load_async<D, BK, 4, kSwzAll>(sK[cur ^ 1], K, (kt + 1) * BK, S, wave, lane);
      tile_load_rows_async<BK, D, 4, kSwzAll>(sV[cur ^ 1], VT + (size_t)(kt + 1) * BK * D, BK, wave, lane);
    }
    const int key0 = kt * BK;
    const bool active = (wrow0 < S) && key0 + BK - 1 >= w_first_min && key0 <= w_last_max;
    if (active) {
      floatx16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b] = floatx16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          mma32(s[b], tile_row_frag<D, kSwzAll>(sK[cur], b * 32 + col, 2 * ks + half), qf[ks]);
      }
      const bool need_mask = key0 < w_first_max || key0 + BK - 1 > w_last_min;
      if (need_mask) {
        // key of register j = key0 + 32b + 4half + kj(j); keep it iff lo <= kj(j) <= hi
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int kb = key0 + b * 32 + half * 4;
          const int lo = kw.first - kb, hi = kw.last - kb;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (c_row(j, 0) < lo || c_row(j, 0) > hi) s[b][j] = NEG_INF;
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
      // Rescale only when some row's max moved (alpha == 1 otherwise: exact skip).
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o_acc[db] *= alpha;
      }
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
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          floatx8 pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = s[b][st * 8 + e];
          const bf16x8 pf = to_frag(pv, bf16());
#pragma unroll
          // V^T row db*32+col, positions 32b + 16st + 8half .. +7: the keys
          // 32b + 16st + c_row(e, half), e = 0..7, in the order of pf
          for (int db = 0; db < NDB; ++db)
            mma32(o_acc[db], tile_row_frag<BK, kSwzAll>(sV[cur], db * 32 + col, 4 * b + 2 * st + half), pf);
        }
    }
    wait_vm();
    __syncthreads();
  }

  const float l_tot = wave_xor32_sum(l_run);
  if (my_row < S) {
    const float inv = 1.f / l_tot;
    bf16* O = p.o + (size_t)hl * head_elems + (size_t)my_row * D;
    bf16* Olo = p.o_lo ? p.o_lo + ((size_t)my_row * p.H + hl) * D : nullptr;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = o_acc[db][jg * 4 + e] * inv;
        const bf16x4 hi = to_out4(o4, bf16());
        *reinterpret_cast<bf16x4*>(O + db * 32 + jg * 8 + half * 4) = hi;
        if (Olo) {
          const floatx4 r = o4 - __builtin_convertvector(hi, floatx4);
          *reinterpret_cast<bf16x4*>(Olo + db * 32 + jg * 8 + half * 4) = to_out4(r, bf16());
        }
      }
    if (half == 0) p.lse[(size_t)hl * S + my_row] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Forward, two wave groups one phase apart: 8 waves x 32 query rows (256 rows
// per workgroup, one workgroup and two waves per SIMD on each CU). Each wave
// runs, per key tile u, an MFMA phase (P V of tile u-1, then the scores of
// tile u) and a softmax phase (mask, row max, rescale, exp, row sum, P to
// bf16), each phase ending at a workgroup barrier. The waves of group 1 pass
// one extra barrier before the tile loop (group 0 one after it), so on every
// SIMD one wave's MFMAs run beside the other wave's softmax VALU work instead
// of both waves reaching the same phase together. All waves run the same
// code; only the position of the extra barrier depends on the group.
// Per row, the operations are those of the 4-wave kernel above (rescale O,
// then add P V, tile by tile); only the row sum of each tile is added in
// four chains instead of one.
// K of tile u lives in sK[u mod 3], V of tile u in sV[u mod 3]. Group 0
// issues the copies of K(u+2) and V(u+1) at the start of its softmax phase
// of tile u and waits for them at the end of its softmax phase of u+1
// (vmcnt leaving only the newer copies in flight), before the barrier after
// which they are first read (its MFMA phase of u+2): two phases of latency.
// The buffers it overwrites (K(u-1), V(u-2)) were last read in the MFMA
// phases of u-1, before the barrier that ends the other group's. The copies
// are untracked by the compiler (lds_copy16x4_untracked), so it keeps
// counting the MFMA phases' LDS reads in order while they are in flight.
// ---------------------------------------------------------------------------
// Scheduling request for a block of N MFMAs that each use R LDS reads: the
// reads of the first AHEAD MFMAs, then one MFMA and R reads at a time, then
// the last AHEAD MFMAs (instruction-scheduler groups; no effect on the
// results).
// The same for N pairs of MFMAs whose operands take R LDS reads per pair,
// AHEAD pairs ahead.
template <int N, int AHEAD, int R>
__device__ __forceinline__ void mfma_pair_ds_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * AHEAD, 0);
}

template <int N, int AHEAD, int R = 1>
__device__ __forceinline__ void mfma_ds_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // its R DS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

template <int D>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_pp_kernel(FwdParams<bf16> p) {
  constexpr int BQ = Bf16Tiles::kFwdPpRows, BK = Bf16Tiles::kFwdKeys, NKS = D / 16, NDB = D / 32;
  static_assert(BQ == 8 * 32 && BK == 64, "8 waves x 32 rows; two 32-key blocks per tile");
  __shared__ __attribute__((aligned(1024))) bf16 sK[3][BK * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV[3][BK * D];
  __shared__ int simd_waves[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Groups by SIMD: the first of the workgroup's waves on a SIMD (SIMD id
  // from the HW_ID register) is in group 0, the second in group 1, so each
  // SIMD holds one wave of each group; the copy slot of a group-0 wave is its
  // SIMD. If the waves are not two per SIMD, groups fall back to waves 0-3
  // and 4-7. Either way each group has four waves with distinct copy slots,
  // so results never depend on the placement, only the overlap does.
  if (tid < 4) simd_waves[tid] = 0;
  __syncthreads();
  const int simd = __builtin_amdgcn_s_getreg((4) | (4 << 6) | ((2 - 1) << 11)) & 3;  // HW_ID[5:4]
  int slot = 0;
  if (lane == 0) slot = atomicAdd(&simd_waves[simd], 1);
  slot = __builtin_amdgcn_readfirstlane(slot);
  __syncthreads();
  const bool by_simd = simd_waves[0] == 2 && simd_waves[1] == 2 && simd_waves[2] == 2 && simd_waves[3] == 2;
  const int grp = by_simd ? slot : wave >> 2;   // wave group
  const int cw = by_simd ? simd : wave & 3;     // copy slot within group 0
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;

  // XCD-aware order as in the 4-wave kernel.
  const int t0 = blockIdx.x;
  const int t = (t0 / 64 + 1) * 64 <= (int)gridDim.x ? (t0 & ~63) | ((t0 & 7) << 3) | ((t0 >> 3) & 7) : t0;
  const int qt = p.causal ? (p.n_qtiles - 1 - t / p.hc) : (t / p.hc);
  const int hl = t % p.hc;
  const int kvl = hl / p.heads_per_kv;
  const size_t head_elems = (size_t)S * D;
  const bf16* __restrict__ Q = p.q + (size_t)hl * head_elems;
  const bf16* __restrict__ K = p.k + (size_t)kvl * head_elems;
  const bf16* __restrict__ VT = p.v + (size_t)kvl * D * p.Sp;

  const int row0 = qt * BQ;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + col;

  const int last_row = min(S, row0 + BQ) - 1;
  const DocSpan kw = key_window(p.doc_off, p.n_docs, min(my_row, S - 1), S, p.causal);
  const int w_first_min = __builtin_amdgcn_readlane(kw.first, 0);
  const int w_first_max = __builtin_amdgcn_readlane(kw.first, 31);
  const int w_last_min = __builtin_amdgcn_readlane(kw.last, 0);
  const int w_last_max = __builtin_amdgcn_readlane(kw.last, 31);
  const int kt_begin = p.doc_off ? key_window(p.doc_off, p.n_docs, row0, S, p.causal).first / BK : 0;
  const int kt_end = key_window(p.doc_off, p.n_docs, last_row, S, p.causal).last / BK + 1;
  const int n_t = kt_end - kt_begin;  // >= 1: a row always sees itself

  // K(0), K(1) and V(0) before the loop; the loop's copies start with K(2), V(1)
  tile_load_async<D, BK, 8, kSwzAll>(sK[0], K, kt_begin * BK, S, wave, lane);
  if (n_t > 1) tile_load_async<D, BK, 8, kSwzAll>(sK[1], K, (kt_begin + 1) * BK, S, wave, lane);
  tile_load_rows_async<BK, D, 8, kSwzAll>(sV[0], VT + (size_t)kt_begin * BK * D, BK, wave, lane);

  bf16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = my_row < S ? *reinterpret_cast<const bf16x8*>(Q + (size_t)my_row * D + ks * 16 + half * 8) : bf16x8{};

  floatx16 o_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o_acc[db] = floatx16{};
  const float NEG_INF = -__builtin_inff();
  float m_run = NEG_INF;
  float l_run = 0.f;
  floatx16 s[2];
  bf16x8 pf[2][2];
  bool s_act = false, p_act = false;

  auto active = [&](int u) {
    const int key0 = (kt_begin + u) * BK;
    return (wrow0 < S) && key0 + BK - 1 >= w_first_min && key0 <= w_last_max;
  };
  // Barrier without a memory fence: LDS reads of the phase done, in-flight
  // tile copies not waited for.
  auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  // One tile: MFMA phase, barrier, softmax phase, barrier.
  // tile u: K(u) in sk, V(u-1) in sv_prev; copies go to sk_next (K(u+2))
  // and sv_dst (V(u+1))
  auto tile = [&](int u, const bf16* sk, const bf16* sv_prev, bf16* sk_next, bf16* sv_dst) {
    // Each MFMA block reads its 16 fragments four MFMAs ahead of their use:
    // in this phase no other wave's MFMAs fill the gaps of an LDS wait.
    if (p_act) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            mma32(o_acc[db], tile_row_frag<BK, kSwzAll>(sv_prev, db * 32 + col, 4 * b + 2 * st + half), pf[b][st]);
      mfma_ds_pipeline<16, 4>();
    }
    s_act = u < n_t && active(u);
    if (s_act) {
      // both 32-key blocks' accumulators live from the first MFMA on
      s[0] = floatx16{};
      s[1] = floatx16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          mma32(s[b], tile_row_frag<D, kSwzAll>(sk, b * 32 + col, 2 * ks + half), qf[ks]);
      mfma_ds_pipeline<16, 4>();
    }
    barrier();
    // the copies of K(u+2) and V(u+1), by group 0
    const bool cp_k = u + 2 < n_t, cp_v = u + 1 < n_t;
    if (grp == 0) {
      if (cp_k) tile_load_untracked<D, BK, 4, kSwzAll>(sk_next, K, (kt_begin + u + 2) * BK, S, cw, lane);
      if (cp_v)
        tile_load_rows_untracked<BK, D, 4, kSwzAll>(sv_dst, VT + (size_t)(kt_begin + u + 1) * BK * D, BK, cw, lane);
    }
    if (s_act) {
      const int key0 = (kt_begin + u) * BK;
      const bool need_mask = key0 < w_first_max || key0 + BK - 1 > w_last_min;
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int kb = key0 + b * 32 + half * 4;
          const int lo = kw.first - kb, hi = kw.last - kb;
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (c_row(j, 0) < lo || c_row(j, 0) > hi) s[b][j] = NEG_INF;
        }
      }
      // The softmax phase runs beside the other group's MFMAs with no other
      // VALU work to fill its latencies: reductions go as independent chains,
      // not one serial chain (the max is exact in any order).
      float mx0 = NEG_INF, mx1 = NEG_INF;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        mx0 = fmaxf(mx0, s[0][j]);
        mx1 = fmaxf(mx1, s[1][j]);
      }
      float mx = wave_xor32_max(fmaxf(mx0, mx1));
      const float m_new = fmaxf(m_run, mx * p.scale_log2);
      const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o_acc[db] *= alpha;
      }
      // row sum in four chains (registers j = 4c + e go to chain e), combined
      // pairwise
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          s[b][j] = __builtin_amdgcn_exp2f(fmaf(s[b][j], p.scale_log2, -m_use));
          ps[j & 3] += s[b][j];
        }
      l_run = l_run * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
      m_run = m_new;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          floatx8 pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = s[b][st * 8 + e];
          pf[b][st] = to_frag(pv, bf16());
        }
    }
    p_act = s_act;
    // the previous tile's copies complete; this tile's (4 per wave for K,
    // 4 for V) may stay in flight. Group 1 has none.
    if (grp == 0) {
      if (cp_k && cp_v)
        wait_vm_leave<8>();
      else if (cp_k || cp_v)
        wait_vm_leave<4>();
      else
        wait_vm_leave<0>();
    }
    barrier();
  };

  wait_vm();
  __syncthreads();
  if (grp == 1) barrier();
  // tiles u = 0 .. n_t (the last one only adds P V of tile n_t - 1)
  int i0 = 0, i1 = 1, i2 = 2;  // u, u + 1, u + 2 mod 3
  for (int u = 0; u <= n_t; ++u) {
    tile(u, sK[i0], sV[i2], sK[i2], sV[i1]);
    const int t_ = i0;
    i0 = i1;
    i1 = i2;
    i2 = t_;
  }
  if (grp == 0) barrier();

  const float l_tot = wave_xor32_sum(l_run);
  if (my_row < S) {
    const float inv = 1.f / l_tot;
    bf16* O = p.o + (size_t)hl * head_elems + (size_t)my_row * D;
    bf16* Olo = p.o_lo ? p.o_lo + ((size_t)my_row * p.H + hl) * D : nullptr;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = o_acc[db][jg * 4 + e] * inv;
        const bf16x4 hi = to_out4(o4, bf16());
        *reinterpret_cast<bf16x4*>(O + db * 32 + jg * 8 + half * 4) = hi;
        if (Olo) {
          const floatx4 r = o4 - __builtin_convertvector(hi, floatx4);
          *reinterpret_cast<bf16x4*>(Olo + db * 32 + jg * 8 + half * 4) = to_out4(r, bf16());
        }
      }
    if (half == 0) p.lse[(size_t)hl * S + my_row] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// dQ: 4 waves x 32 query rows, 64-key tiles, one 32-key block at a time.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_bf16_kernel(BwdParams<bf16> p) {
  constexpr int BQ = Bf16Tiles::kDqRows, BK = Bf16Tiles::kDqKeys, NKS = D / 16, NDB = D / 32;
  static_assert(BQ == 4 * 32 && BK == 64, "4 waves x 32 rows; two 32-key blocks per tile");
  __shared__ __attribute__((aligned(1024))) bf16 sK[2][BK * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV[2][BK * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;

  // XCD-aware order, as in the forward.
  const int t0 = blockIdx.x;
  const int t = (t0 / 64 + 1) * 64 <= (int)gridDim.x ? (t0 & ~63) | ((t0 & 7) << 3) | ((t0 >> 3) & 7) : t0;
  const int qt = p.causal ? (p.n_qtiles - 1 - t / p.hc) : (t / p.hc);
  const int hl = t % p.hc;
  const int kvl = hl / p.heads_per_kv;
  const size_t head_elems = (size_t)S * D;
  const bf16* __restrict__ Q = p.q + (size_t)hl * head_elems;
  const bf16* __restrict__ dO = p.dout + (size_t)hl * head_elems;
  const bf16* __restrict__ K = p.k + (size_t)kvl * head_elems;
  const bf16* __restrict__ V = p.v + (size_t)kvl * head_elems;

  const int row0 = qt * BQ;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + col;
  const bool row_ok = my_row < S;

  // Key windows as in the forward kernel.
  const int last_row = min(S, row0 + BQ) - 1;
  const DocSpan kw = key_window(p.doc_off, p.n_docs, min(my_row, S - 1), S, p.causal);
  const int w_first_min = __builtin_amdgcn_readlane(kw.first, 0);
  const int w_first_max = __builtin_amdgcn_readlane(kw.first, 31);
  const int w_last_min = __builtin_amdgcn_readlane(kw.last, 0);
  const int w_last_max = __builtin_amdgcn_readlane(kw.last, 31);
  const int kt_begin = p.doc_off ? key_window(p.doc_off, p.n_docs, row0, S, p.causal).first / BK : 0;
  const int kt_end = key_window(p.doc_off, p.n_docs, last_row, S, p.causal).last / BK + 1;

  tile_load_async<D, BK, 4>(sK[kt_begin & 1], K, kt_begin * BK, S, wave, lane);
  tile_load_async<D, BK, 4>(sV[kt_begin & 1], V, kt_begin * BK, S, wave, lane);

  bf16x8 qf[NKS], df[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + (size_t)my_row * D + ks * 16 + half * 8) : bf16x8{};
    df[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(dO + (size_t)my_row * D + ks * 16 + half * 8) : bf16x8{};
  }
  const float l2 = row_ok ? p.lse2[(size_t)hl * S + my_row] : 0.f;
  const float nD = row_ok ? p.negD[(size_t)hl * S + my_row] : 0.f;

  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};

  wait_vm();
  __syncthreads();
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < kt_end) {
      tile_load_async<D, BK, 4>(sK[cur ^ 1], K, (kt + 1) * BK, S, wave, lane);
      tile_load_async<D, BK, 4>(sV[cur ^ 1], V, (kt + 1) * BK, S, wave, lane);
    }
    const int key0 = kt * BK;
    const bool active = (wrow0 < S) && key0 + BK - 1 >= w_first_min && key0 <= w_last_max;
    if (active) {
      const bool need_mask = key0 < w_first_max || key0 + BK - 1 > w_last_min;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        // dP starts from this lane's row -D, so the MFMAs yield dP - D
        floatx16 s = floatx16{}, dp;
#pragma unroll
        for (int j = 0; j < 16; ++j) dp[j] = nD;
        // MFMA runs at raised wave priority, so the SIMD's other wave (in
        // its softmax) does not delay the MFMA issue stream.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          mma32(s, tile_row_frag<D>(sK[cur], b * 32 + col, 2 * ks + half), qf[ks]);
          mma32(dp, tile_row_frag<D>(sV[cur], b * 32 + col, 2 * ks + half), df[ks]);
        }
        __builtin_amdgcn_s_setprio(0);
        if (need_mask) {
          // key of register j = key0 + 32b + 4half + kj(j); keep it iff lo <= kj(j) <= hi
          const int kb = key0 + b * 32 + half * 4;
          const int lo = kw.first - kb, hi = kw.last - kb;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int kj = c_row(j, 0);
            const float pij = (kj >= lo && kj <= hi) ? __builtin_amdgcn_exp2f(fmaf(s[j], p.scale_log2, -l2)) : 0.f;
            s[j] = pij * dp[j];  // dS^T = P (dP - D)
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float pij = __builtin_amdgcn_exp2f(fmaf(s[j], p.scale_log2, -l2));
            s[j] = pij * dp[j];  // dS^T = P (dP - D)
          }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          floatx8 d8;
#pragma unroll
          for (int e = 0; e < 8; ++e) d8[e] = s[st * 8 + e];
          const bf16x8 dsf = to_frag(d8, bf16());
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            mma32(acc[db], tile_tr_frag<D>(sK[cur], b * 32 + st * 16, db * 32, lane), dsf);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    wait_vm();
    __syncthreads();
  }

  if (row_ok) {
    bf16* dQ = p.dq + (size_t)hl * head_elems + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[db][jg * 4 + e] * p.scale;
        *reinterpret_cast<bf16x4*>(dQ + db * 32 + jg * 8 + half * 4) = to_out4(v4, bf16());
      }
  }
}

// ---------------------------------------------------------------------------
// dQ, two wave groups one phase apart (the scheme of the two-group forward):
// 8 waves x 32 query rows, 256 rows per workgroup, key tiles of 32 (one
// block per phase keeps the scores, dP - D and dS of a tile within the
// register budget). Per key tile u, the MFMA phase adds dS(u-1) K(u-1) to
// dQ and forms the scores and dP - D of tile u; the softmax phase turns them
// into dS(u) = P (dP - D) in bf16. dQ receives the same products in the same
// order as in the 4-wave kernel above (16-key steps in key order), so
// results are identical.
// K of tile u lives in sK[u mod 4] (it is read again, transposed, in the MFMA
// phase of u+1), V of tile u in sV[u mod 3]. In its softmax phase of u, group
// 0 copies K(u+2) (its waves 0-1) and V(u+2) (waves 2-3) and waits for them
// at the end of its softmax phase of u+1; they are first read in its MFMA
// phase of u+2. The buffers they overwrite (K(u-2), V(u-1)) were last read in
// the MFMA phases of u-1. The copies are untracked (lds_copy16x4_untracked).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_bf16_pp_kernel(BwdParams<bf16> p) {
  constexpr int BQ = Bf16Tiles::kDqPpRows, BK = Bf16Tiles::kDqPpKeys, NKS = D / 16, NDB = D / 32;
  static_assert(BQ == 8 * 32 && BK == 32, "8 waves x 32 rows; one 32-key block per tile");
  __shared__ __attribute__((aligned(1024))) bf16 sK[4][BK * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV[3][BK * D];
  __shared__ int simd_waves[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave groups by SIMD, as in the two-group forward
  if (tid < 4) simd_waves[tid] = 0;
  __syncthreads();
  const int simd = __builtin_amdgcn_s_getreg((4) | (4 << 6) | ((2 - 1) << 11)) & 3;  // HW_ID[5:4]
  int slot = 0;
  if (lane == 0) slot = atomicAdd(&simd_waves[simd], 1);
  slot = __builtin_amdgcn_readfirstlane(slot);
  __syncthreads();
  const bool by_simd = simd_waves[0] == 2 && simd_waves[1] == 2 && simd_waves[2] == 2 && simd_waves[3] == 2;
  const int grp = by_simd ? slot : wave >> 2;
  const int cw = by_simd ? simd : wave & 3;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;

  const int t0 = blockIdx.x;
  const int t = (t0 / 64 + 1) * 64 <= (int)gridDim.x ? (t0 & ~63) | ((t0 & 7) << 3) | ((t0 >> 3) & 7) : t0;
  const int qt = p.causal ? (p.n_qtiles - 1 - t / p.hc) : (t / p.hc);
  const int hl = t % p.hc;
  const int kvl = hl / p.heads_per_kv;
  const size_t head_elems = (size_t)S * D;
  const bf16* __restrict__ Q = p.q + (size_t)hl * head_elems;
  const bf16* __restrict__ dO = p.dout + (size_t)hl * head_elems;
  const bf16* __restrict__ K = p.k + (size_t)kvl * head_elems;
  const bf16* __restrict__ V = p.v + (size_t)kvl * head_elems;

  const int row0 = qt * BQ;
  const int wrow0 = row0 + wave * 32;
  const int my_row = wrow0 + col;
  const bool row_ok = my_row < S;

  const int last_row = min(S, row0 + BQ) - 1;
  const DocSpan kw = key_window(p.doc_off, p.n_docs, min(my_row, S - 1), S, p.causal);
  const int w_first_min = __builtin_amdgcn_readlane(kw.first, 0);
  const int w_first_max = __builtin_amdgcn_readlane(kw.first, 31);
  const int w_last_min = __builtin_amdgcn_readlane(kw.last, 0);
  const int w_last_max = __builtin_amdgcn_readlane(kw.last, 31);
  const int kt_begin = p.doc_off ? key_window(p.doc_off, p.n_docs, row0, S, p.causal).first / BK : 0;
  const int kt_end = key_window(p.doc_off, p.n_docs, last_row, S, p.causal).last / BK + 1;
  const int n_t = kt_end - kt_begin;

  // K(0), V(0), K(1), V(1) before the loop; the loop's copies start with tile 2
  tile_load_async<D, BK, 8>(sK[0], K, kt_begin * BK, S, wave, lane);
  tile_load_async<D, BK, 8>(sV[0], V, kt_begin * BK, S, wave, lane);
  if (n_t > 1) {
    tile_load_async<D, BK, 8>(sK[1], K, (kt_begin + 1) * BK, S, wave, lane);
    tile_load_async<D, BK, 8>(sV[1], V, (kt_begin + 1) * BK, S, wave, lane);
  }

  bf16x8 qf[NKS], df[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + (size_t)my_row * D + ks * 16 + half * 8) : bf16x8{};
    df[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(dO + (size_t)my_row * D + ks * 16 + half * 8) : bf16x8{};
  }
  const float l2 = row_ok ? p.lse2[(size_t)hl * S + my_row] : 0.f;
  const float nD = row_ok ? p.negD[(size_t)hl * S + my_row] : 0.f;

  floatx16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = floatx16{};
  floatx16 s, dp;
  bf16x8 dsf[2];
  bool s_act = false, ds_act = false;

  auto active = [&](int u) {
    const int key0 = (kt_begin + u) * BK;
    return (wrow0 < S) && key0 + BK - 1 >= w_first_min && key0 <= w_last_max;
  };
  auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  // tile u: K(u) in sk, K(u-1) in sk_prev, V(u) in sv; copies of K(u+2), V(u+2)
  // go to sk_dst, sv_dst
  auto tile = [&](int u, const bf16* sk, const bf16* sk_prev, const bf16* sv, bf16* sk_dst, bf16* sv_dst) {
    if (ds_act) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          mma32(acc[db], tile_tr_frag<D>(sk_prev, st * 16, db * 32, lane), dsf[st]);
      mfma_ds_pipeline<8, 2, 2>();
    }
    s_act = u < n_t && active(u);
    if (s_act) {
      // dP starts from this lane's row -D, so the MFMAs yield dP - D
      s = floatx16{};
#pragma unroll
      for (int j = 0; j < 16; ++j) dp[j] = nD;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        mma32(s, tile_row_frag<D>(sk, col, 2 * ks + half), qf[ks]);
        mma32(dp, tile_row_frag<D>(sv, col, 2 * ks + half), df[ks]);
      }
      mfma_ds_pipeline<16, 4>();
    }
    barrier();
    const bool cp = u + 2 < n_t;
    if (grp == 0 && cp) {
      if (cw < 2)
        tile_load_untracked<D, BK, 2>(sk_dst, K, (kt_begin + u + 2) * BK, S, cw, lane);
      else
        tile_load_untracked<D, BK, 2>(sv_dst, V, (kt_begin + u + 2) * BK, S, cw - 2, lane);
    }
    if (s_act) {
      const int key0 = (kt_begin + u) * BK;
      const bool need_mask = key0 < w_first_max || key0 + BK - 1 > w_last_min;
      if (need_mask) {
        const int kb = key0 + half * 4;
        const int lo = kw.first - kb, hi = kw.last - kb;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kj = c_row(j, 0);
          const float pij = (kj >= lo && kj <= hi) ? __builtin_amdgcn_exp2f(fmaf(s[j], p.scale_log2, -l2)) : 0.f;
          s[j] = pij * dp[j];  // dS^T = P (dP - D)
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pij = __builtin_amdgcn_exp2f(fmaf(s[j], p.scale_log2, -l2));
          s[j] = pij * dp[j];
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 d8;
#pragma unroll
        for (int e = 0; e < 8; ++e) d8[e] = s[st * 8 + e];
        dsf[st] = to_frag(d8, bf16());
      }
    }
    ds_act = s_act;
    // the previous tile's copies complete; this tile's (4 per wave) may stay
    // in flight. Group 1 has none.
    if (grp == 0) {
      if (cp)
        wait_vm_leave<4>();
      else
        wait_vm_leave<0>();
    }
    barrier();
  };

  wait_vm();
  __syncthreads();
  if (grp == 1) barrier();
  int k0 = 0, k3 = 3, k2 = 2;  // u, u - 1, u + 2 mod 4
  int v0 = 0, v2 = 2;          // u, u + 2 mod 3
  for (int u = 0; u <= n_t; ++u) {
    tile(u, sK[k0], sK[k3], sV[v0], sK[k2], sV[v2]);
    k3 = k0;
    k0 = (k0 + 1) & 3;
    k2 = (k2 + 1) & 3;
    v0 = v0 == 2 ? 0 : v0 + 1;
    v2 = v2 == 2 ? 0 : v2 + 1;
  }
  if (grp == 0) barrier();

  if (row_ok) {
    bf16* dQ = p.dq + (size_t)hl * head_elems + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[db][jg * 4 + e] * p.scale;
        *reinterpret_cast<bf16x4*>(dQ + db * 32 + jg * 8 + half * 4) = to_out4(v4, bf16());
      }
  }
}

// ---------------------------------------------------------------------------
// dK/dV: 4 waves x 32 keys; query rows in steps of 32, head-major, each head's
// row blocks from the last one down to the workgroup's diagonal. Workgroups
// resident together then read the same Q/dO block at about the same time, so
// it is fetched once per L2 instead of once per workgroup.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_bf16_kernel(BwdParams<bf16> p) {
  constexpr int BKV = Bf16Tiles::kDkvKeys, BQ = Bf16Tiles::kDkvRows, NKS = D / 16, NDB = D / 32;
  static_assert(BKV == 4 * 32 && BQ == 32, "4 waves x 32 keys; 32-row steps");
  // These tiles use the layout with both read kinds conflict-free (kSwzAll):
  // this kernel issues the most LDS reads per MFMA.
  __shared__ __attribute__((aligned(1024))) bf16 sQ[2][BQ * D];
  __shared__ __attribute__((aligned(1024))) bf16 sO[2][BQ * D];  // dO rows
  __shared__ __attribute__((aligned(256))) float sLD[2][2 * BQ];  // lse*log2(e) | -D
  __shared__ __attribute__((aligned(1024))) bf16 sV[BKV * D];     // this workgroup's V rows

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;

  // XCD-aware order, as in the forward: each XCD takes runs of 8 consecutive
  // key tiles, which walk the same query blocks.
  const int t0 = blockIdx.x;
  const int t = (t0 / 64 + 1) * 64 <= (int)gridDim.x ? (t0 & ~63) | ((t0 & 7) << 3) | ((t0 >> 3) & 7) : t0;
  const int kt = t / p.nkv;
  const int g = t % p.nkv;
  const size_t head_elems = (size_t)S * D;
  const bf16* __restrict__ K = p.k + (size_t)g * head_elems;
  const bf16* __restrict__ V = p.v + (size_t)g * head_elems;

  const int key0 = kt * BKV;
  const int wkey0 = key0 + wave * 32;
  const int my_key = wkey0 + col;
  const bool key_ok = my_key < S;

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

  // Step order: head hi ascending, row block qb from qb_top down to qb0.
  // (hi, qb) cursors advance by compare-and-select instead of dividing the
  // step index each step.
  auto advance = [&](int& hi, int& qb) {
    if (qb == qb0) {
      qb = qb_top;
      ++hi;
    } else {
      --qb;
    }
  };
  // The step copies are untracked (lds_copy16x2_untracked): the compiler
  // would otherwise wait for the next step's copies before the first LDS
  // read of the current step. They are waited for at the end of the step.
  auto issue = [&](int hi, int qb, int buf) {
    const int hl = g * p.heads_per_kv + hi;
    const int r0 = qb * BQ;
    tile_load_untracked<D, BQ, 4, kSwzAll>(sQ[buf], p.q + (size_t)hl * head_elems, r0, S, wave, lane);
    tile_load_untracked<D, BQ, 4, kSwzAll>(sO[buf], p.dout + (size_t)hl * head_elems, r0, S, wave, lane);
    if (wave == 0) {
      const int r = min(r0 + (lane & 31), S - 1);
      const float* src = (lane < 32 ? p.lse2 : p.negD) + (size_t)hl * S + r;
      lds_copy4_untracked((const void*)src, (lds_void*)&sLD[buf][0]);
    }
  };

  // V^T operand of dP = dO V^T stays in LDS (read per step); K^T stays in
  // registers: both together would not fit two waves per SIMD.
  tile_load_async<D, BKV, 4, kSwzAll>(sV, V, key0, S, wave, lane);
  int next_hi = 0, next_qb = qb_top;  // the next step to copy in
  int cur_qb = qb_top;                // the step being computed
  int cur_hi = 0;
  issue(next_hi, next_qb, 0);
  advance(next_hi, next_qb);

  bf16x8 kf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kf[ks] = key_ok ? *reinterpret_cast<const bf16x8*>(K + (size_t)my_key * D + ks * 16 + half * 8) : bf16x8{};

  floatx16 dk[NDB], dv[NDB];
  if (p.acc_load) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const size_t off = (size_t)g * head_elems + (size_t)my_key * D + db * 32 + jg * 8 + half * 4;
        const floatx4 a = key_ok ? *reinterpret_cast<const floatx4*>(p.dk_acc + off) : floatx4{};
        const floatx4 b = key_ok ? *reinterpret_cast<const floatx4*>(p.dv_acc + off) : floatx4{};
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

  wait_vm();
  __syncthreads();
  for (int step = 0; step < n_steps; ++step) {
    const int cur = step & 1;
    if (step + 1 < n_steps) {
      issue(next_hi, next_qb, cur ^ 1);
      advance(next_hi, next_qb);
      // Every fourth step the copy just issued is waited for at once. A
      // workgroup that has run ahead of the others sharing its Q/dO blocks
      // misses in L2 and pays that latency here, which holds it back to
      // them; without this they drift apart over long walks (several heads
      // per chunk) and fetch far more from beyond L2.
      if ((step & 3) == 0) wait_vm();
    }
    const int r0 = cur_qb * BQ;
    const bool active = (wkey0 < S) && r0 + BQ - 1 >= w_first_min && r0 <= w_last_max;
    if (active) {
      // dP starts from -D of each row (register j: row r0 + 4half + kj(j)), so
      // the MFMAs produce dP - D directly.
      floatx16 s = floatx16{}, dp;
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(&sLD[cur][BQ + jg * 8 + half * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[jg * 4 + e] = d4[e];
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        mma32(s, tile_row_frag<D, kSwzAll>(sQ[cur], col, 2 * ks + half), kf[ks]);
        mma32(dp, tile_row_frag<D, kSwzAll>(sO[cur], col, 2 * ks + half), tile_row_frag<D, kSwzAll>(sV, wave * 32 + col, 2 * ks + half));
      }
      // fragments read ahead of their MFMAs (three reads per pair)
      mfma_pair_ds_pipeline<NKS, 2, 3>();
      __builtin_amdgcn_s_setprio(0);
      const bool need_mask = r0 < w_first_max || r0 + BQ - 1 > w_last_min;
      if (need_mask) {
        // row of register j = r0 + 4half + kj(j); it counts iff lo <= kj(j) <= hi.
        // Excluded scores become -inf, so their exp2 below is exactly 0.
        const int rb = r0 + half * 4;
        const int lo = rw.first - rb;
        const int hi = rw.last - rb;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kj = c_row(j, 0);
          if (kj < lo || kj > hi) s[j] = -__builtin_inff();
        }
      }
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(&sLD[cur][jg * 8 + half * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jg * 4 + e;
          const float pij = __builtin_amdgcn_exp2f(fmaf(s[j], p.scale_log2, -l4[e]));
          s[j] = pij;
          dp[j] = pij * dp[j];  // dS = P (dP - D)
        }
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        floatx8 p8, d8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p8[e] = s[st * 8 + e];
          d8[e] = dp[st * 8 + e];
        }
        const bf16x8 pf = to_frag(p8, bf16());
        const bf16x8 dsf = to_frag(d8, bf16());
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          mma32(dv[db], tile_tr_frag<D, kSwzAll>(sO[cur], st * 16, db * 32, lane), pf);
          mma32(dk[db], tile_tr_frag<D, kSwzAll>(sQ[cur], st * 16, db * 32, lane), dsf);
        }
      }
      // two transposed reads per MFMA, two MFMAs ahead
      mfma_ds_pipeline<2 * 2 * NDB, 2, 2>();
      __builtin_amdgcn_s_setprio(0);
    }
    advance(cur_hi, cur_qb);
    wait_vm();
    __syncthreads();
  }

  if (!key_ok) return;
  if (p.finalize) {
    bf16* dK = p.dk_out + ((size_t)my_key * p.Hkv_total + g) * D;
    bf16* dV = p.dv_out + ((size_t)my_key * p.Hkv_total + g) * D;
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
        *reinterpret_cast<bf16x4*>(dK + db * 32 + jg * 8 + half * 4) = to_out4(a, bf16());
        *reinterpret_cast<bf16x4*>(dV + db * 32 + jg * 8 + half * 4) = to_out4(b, bf16());
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
