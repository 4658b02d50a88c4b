// The fused deterministic backward for bf16 heads of 128: one kv-major kernel
// computes dK, dV and dQ from a single pass over every (row block, key tile)
// pair, so the scores S = Q K^T and dP = dO V^T are formed once per pair
// instead of once in a dK/dV kernel and again in a dQ kernel (five products
// per pair instead of seven). It is the backward pass of the attention that
// the head chunks run ("Road to 5 Million Tokens" talk summary, Chapters: the
// activation-checkpointing chapter, on recomputing in the backward rather
// than storing the S-long intermediates), with the same gradients as the
// two-kernel backward and the same results on every run.
//
// dQ of a row block is a sum over key tiles, and key tiles belong to
// different workgroups. Floating-point sums depend on their order, so the
// order is fixed:
//  * key tile kt belongs to XCD kt mod nx (nx = the device's XCD count), and
//    each XCD keeps its own fp32 dQ partial [hc][S][128] in the workspace.
//    Every workgroup that adds into partial x runs on XCD x, so all of them
//    share that XCD's L2: a store that has completed is seen by the next
//    reader on that XCD whose load skips its CU's L1 (sc0), and no L2
//    write-back is needed;
//  * the tiles of an XCD are handed out by a per-XCD ticket counter in
//    ascending kt (the heaviest causal tiles first), and tile kt adds its
//    terms to a 32-row block only after tile kt - nx has added its own: per
//    wave (each wave owns 32 of the 128 dQ columns) a progress word counts
//    the steps whose additions have completed, stored once those stores have
//    completed (into the XCD's L2) and read by the next tile through the
//    scalar unit with the scalar cache bypassed;
//  * a final kernel adds the nx partials in ascending x.
// The tile a workgroup waits for holds an earlier ticket of the same queue,
// so it was taken by a workgroup that is already running: the lowest
// unfinished ticket of each queue never waits, and every wait ends. Each wait
// also has a poll limit; when it runs out the call records an error, later
// waits stop waiting, and the final kernel writes NaN to all of dQ.
//
// Tiles walk their row blocks upward from the diagonal, so consecutive tiles
// of a queue meet the same row block one step apart: the partial rows one
// tile has just written are still in L2 for the next, and so are the Q and dO
// rows they both read.
#pragma once

#include "attn_bf16.hpp"

namespace upipe {

struct FusedSync {
  float* partial;  // [nx][hc][S][128] fp32; rows a queue's first tile does not cover are never read
  int* tickets;    // [nx] next ticket of each XCD's queue, zero at launch
  int* progress;   // [n_ktiles][nkv][4] completed-step count of each (tile, wave), zero at launch
  int* error;      // zero at launch; set when a wait runs out of polls
  int nx;          // XCDs of the device
  int max_polls;   // polls per wait before giving up
};

// The dS tile of one step: [128 keys][32 rows] bf16, 64-byte key rows; the
// 8-byte slot s (rows 4s .. 4s+3) of key k sits at slot s ^ ((k >> 2) & 7).
// Eight-byte writes of 32 consecutive keys and the transposed reads of four
// consecutive keys then both touch 32 different bank pairs.
__device__ __forceinline__ int dstile_off(int key, int slot) { return key * 32 + ((slot ^ ((key >> 2) & 7)) << 2); }

// Operand fragment of dS with the contraction over keys: lane (m, half)
// receives dS[row m][key rbase + c_row(e, half)], e = 0..7 (the k order of
// tile_tr_frag, which reads the matching K^T fragment).
__device__ __forceinline__ bf16x8 dstile_frag(const bf16* t, int rbase, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int key = rbase + ((g >> 1) << 2) + (j >> 2);
  const int slot = ((g & 1) << 2) + (j & 3);
  const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(t + dstile_off(key, slot)));
  const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(t + dstile_off(key + 8, slot)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Wait until at most n (0, 4 or 5) of this wave's vector memory operations
// are outstanding.
__device__ __forceinline__ void wait_vm_leave_n(int n) {
  if (n == 5)
    __builtin_amdgcn_s_waitcnt(0x0F70 | 5);
  else if (n == 4)
    __builtin_amdgcn_s_waitcnt(0x0F70 | 4);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The value itself, hidden from the optimizer: LDS addresses derived from it
// are recomputed where they are used instead of being held in registers
// across the whole step loop (which would not fit two waves per SIMD).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// A progress word read through the scalar unit with the scalar cache
// bypassed, so it comes from the XCD's L2, where its writer (a workgroup of
// the same XCD, with an ordinary store) put it. A vector load would also have to wait for this wave's
// global->LDS copies in flight (they share one counter); this wait counts LDS
// and scalar operations only. The address must be the same in every lane.
__device__ __forceinline__ int poll_word(const int* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Workgroup barrier after this wave's LDS accesses have completed; outstanding
// global memory operations are left in flight (the callers wait for the ones
// they need by count).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 4 waves x 32 keys, 32-row steps, as the dK/dV kernel, plus per step:
// dS to LDS, dQ^T (32 d x 32 rows per wave) = K^T dS^T on top of the
// partial's current rows, written back. K stays in LDS (read as rows for
// S^T and transposed for dQ); V, only read as rows, stays in registers.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_fused_bf16_kernel(BwdParams<bf16> p, FusedSync fs) {
  constexpr int BKV = Bf16Tiles::kDkvKeys, BQ = Bf16Tiles::kDkvRows, NKS = D / 16, NDB = D / 32;
  static_assert(D == 128 && BKV == 4 * 32 && BQ == 32, "4 waves x 32 keys and 32 dQ columns; 32-row steps");
  __shared__ __attribute__((aligned(1024))) bf16 sQ[2][BQ * D];
  __shared__ __attribute__((aligned(1024))) bf16 sO[2][BQ * D];   // dO rows
  __shared__ __attribute__((aligned(256))) float sLD[2][2 * BQ];  // lse*log2(e) | -D
  __shared__ __attribute__((aligned(1024))) bf16 sK[BKV * D];     // this tile's K rows
  __shared__ __attribute__((aligned(1024))) bf16 sDS[BKV * BQ];   // this step's dS
  __shared__ int sTicket;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;
  const size_t head_elems = (size_t)S * D;
  const int nqb = (S + BQ - 1) / BQ;  // row blocks per head; the step code of (hi, qb) is hi * nqb + qb

  // This workgroup's XCD (hardware register XCC_ID) picks its queue.
  const int x = (__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15) % fs.nx;
  const int n_kt_x = x < p.n_ktiles ? (p.n_ktiles - 1 - x) / fs.nx + 1 : 0;
  const int n_tickets = n_kt_x * p.nkv;

  for (;;) {
    if (tid == 0) sTicket = __hip_atomic_fetch_add(&fs.tickets[x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int ticket = __builtin_amdgcn_readfirstlane(sTicket);  // uniform: tile values live in SGPRs
    if (ticket >= n_tickets) break;
    const int kt = x + fs.nx * (ticket / p.nkv);
    const int g = ticket % p.nkv;
    const bf16* __restrict__ K = p.k + (size_t)g * head_elems;
    const bf16* __restrict__ V = p.v + (size_t)g * head_elems;

    const int key0 = kt * BKV;
    const int wkey0 = key0 + wave * 32;
    const int my_key = wkey0 + col;
    const bool key_ok = my_key < S;

    DocSpan rw = row_window(nullptr, 0, min(my_key, S - 1), S, p.causal);
    if (p.causal) rw.first = my_key;
    const int w_first_min = __builtin_amdgcn_readlane(rw.first, 0);
    const int w_first_max = __builtin_amdgcn_readlane(rw.first, 31);
    const int w_last_min = __builtin_amdgcn_readlane(rw.last, 0);
    const int w_last_max = __builtin_amdgcn_readlane(rw.last, 31);
    const int qb0 = p.causal ? key0 / BQ : 0;
    const int qb_top = nqb - 1;
    const int n_steps = p.heads_per_kv * (qb_top - qb0 + 1);

    // Progress words: this wave's, and the same wave's of tile kt - nx (the
    // previous tile of this queue), which covers every row block of this one.
    int* const mine = fs.progress + ((size_t)kt * p.nkv + g) * 4 + wave;
    const int* const pred = kt >= fs.nx ? fs.progress + ((size_t)(kt - fs.nx) * p.nkv + g) * 4 + wave : nullptr;

    // Step order: head hi ascending, row block qb from qb0 up to qb_top.
    // (Both cursors are assigned on every call: a branch that updated one
    // or the other would let the compiler keep them in scratch memory.)
    auto advance = [&](int& hi, int& qb) {
      const bool wrap = qb == qb_top;
      hi += wrap ? 1 : 0;
      qb = wrap ? qb0 : qb + 1;
    };
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
    const int copies_per_step = wave == 0 ? 5 : 4;

    tile_load_async<D, BKV, 4, kSwzAll>(sK, K, key0, S, wave, lane);
    int next_hi = 0, next_qb = qb0;
    int cur_hi = 0, cur_qb = qb0;
    issue(next_hi, next_qb, 0);
    advance(next_hi, next_qb);

    bf16x8 vf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      vf[ks] = key_ok ? *reinterpret_cast<const bf16x8*>(V + (size_t)my_key * D + ks * 16 + half * 8) : bf16x8{};

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
    int done_code = -1;  // step code of the last step whose additions were issued
    for (int step = 0; step < n_steps; ++step) {
      const int cur = step & 1;
      const int lane = opaque(tid & 63);
      const int col = lane & 31, half = lane >> 5;
      int in_flight = 0;  // copies issued in this step
      if (step + 1 < n_steps) {
        issue(next_hi, next_qb, cur ^ 1);
        advance(next_hi, next_qb);
        in_flight = copies_per_step;
      }
      const int r0 = cur_qb * BQ;
      const bool active = (wkey0 < S) && r0 + BQ - 1 >= w_first_min && r0 <= w_last_max;
      floatx16 s = floatx16{}, dp;
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(&sLD[cur][BQ + jg * 8 + half * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[jg * 4 + e] = d4[e];
      }
      if (active) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          mma32(s, tile_row_frag<D, kSwzAll>(sQ[cur], col, 2 * ks + half),
                tile_row_frag<D, kSwzAll>(sK, wave * 32 + col, 2 * ks + half));
          mma32(dp, tile_row_frag<D, kSwzAll>(sO[cur], col, 2 * ks + half), vf[ks]);
        }
        mfma_pair_ds_pipeline<NKS, 2, 3>();
        __builtin_amdgcn_s_setprio(0);
      }

      // The previous step's partial stores were issued before this step's
      // copies: once only the copies may be outstanding, they have completed
      // in L2 and the next tile of the queue may read them.
      if (done_code >= 0) {
        wait_vm_leave_n(in_flight);
        asm volatile("" ::: "memory");
        if (lane == 0) __hip_atomic_store(mine, done_code + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      bf16x8 pf[2], dsf[2];
      if (active) {
        const bool need_mask = r0 < w_first_max || r0 + BQ - 1 > w_last_min;
        if (need_mask) {
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
            dp[j] = key_ok ? pij * dp[j] : 0.f;  // dS = P (dP - D); keys past S add nothing to dQ
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
          pf[st] = to_frag(p8, bf16());
          dsf[st] = to_frag(d8, bf16());
        }
      } else {
        pf[0] = pf[1] = dsf[0] = dsf[1] = bf16x8{};
      }
      const int code = cur_hi * nqb + cur_qb;
      const int hl = g * p.heads_per_kv + cur_hi;
      const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
          fs.partial + ((size_t)x * p.hc + hl) * head_elems, 0, (int)(head_elems * 4u), 0x00020000);
      const unsigned poff = (unsigned)((r0 + col) * D + wave * 32 + half * 4) * 4u;
      floatx16 dq = floatx16{};
      if (pred) {
        // Wait for the previous tile's additions to these rows, then start
        // from the partial's current rows (the loads fly during dV, dK).
        int polls = 0;
        while (poll_word(pred) <= code) {
          if (__hip_atomic_load(fs.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 ||
              ++polls >= fs.max_polls) {
            if (lane == 0) __hip_atomic_store(fs.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const floatx4 v = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(part, poff + jg * 32, 0, 1));
#pragma unroll
          for (int e = 0; e < 4; ++e) dq[jg * 4 + e] = v[e];
        }
      }

      // dS^T of this wave's 32 keys into the step's dS tile: register group
      // st holds rows 16st + 4half + 0..3 and 16st + 8 + 4half + 0..3.
      {
        const int key = wave * 32 + col;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x4 lo4 = __builtin_shufflevector(dsf[st], dsf[st], 0, 1, 2, 3);
          const bf16x4 hi4 = __builtin_shufflevector(dsf[st], dsf[st], 4, 5, 6, 7);
          *reinterpret_cast<bf16x4*>(sDS + dstile_off(key, 4 * st + half)) = lo4;
          *reinterpret_cast<bf16x4*>(sDS + dstile_off(key, 4 * st + 2 + half)) = hi4;
        }
      }
      if (active) {
        const int lane_v = opaque(lane);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            mma32(dv[db], tile_tr_frag<D, kSwzAll>(sO[cur], st * 16, db * 32, lane_v), pf[st]);
            mma32(dk[db], tile_tr_frag<D, kSwzAll>(sQ[cur], st * 16, db * 32, lane_v), dsf[st]);
          }
        mfma_ds_pipeline<2 * 2 * NDB, 2, 2>();
        __builtin_amdgcn_s_setprio(0);
      }
      lds_barrier();  // every wave's dS is in the tile
      const int lane_q = opaque(lane);

      // dQ^T of the wave's 32 columns: lane = row r0 + col, register j =
      // column 32 wave + c_row(j, half); added on top of the partial.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < BKV / 16; ++ks)
        mma32(dq, tile_tr_frag<D, kSwzAll>(sK, 16 * ks, wave * 32, lane_q), dstile_frag(sDS, 16 * ks, lane_q));
      mfma_ds_pipeline<BKV / 16, 2, 4>();
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dq[jg * 4 + e];
        // rows past S fall outside the buffer's range and are dropped
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), part, poff + jg * 32, 0, 1);
      }
      done_code = code;
      advance(cur_hi, cur_qb);
      wait_vm_leave<4>();  // this step's copies (the partial stores may still be in flight)
      lds_barrier();
    }
    wait_vm();
    asm volatile("" ::: "memory");
    if (lane == 0 && done_code >= 0)
      __hip_atomic_store(mine, done_code + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);

    if (key_ok) {
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
    __syncthreads();  // sTicket and the LDS tiles are reused by the next tile
  }
}

// dQ = tau * (partial_0 + partial_1 + ... ) in ascending XCD order, written
// as bf16 into the caller's [S][Hq][128] at the chunk's first head. Partial x
// holds rows from x * 128 on when causal (its queue's first tile, kt = x,
// covers them and starts from zero), all rows otherwise, and nothing when
// x >= n_ktiles. Every value is NaN if a wait gave up or a queue was not
// drained.
__global__ __launch_bounds__(256) void fused_dq_reduce_kernel(const float* __restrict__ partial,
                                                              const int* __restrict__ tickets,
                                                              const int* __restrict__ error, bf16* __restrict__ dq,
                                                              int64_t tok_stride, int S, int hc, int nx, int n_ktiles,
                                                              int nkv, int causal, float scale) {
  constexpr int D = 128, BKV = Bf16Tiles::kDkvKeys;
  bool bad = error[0] != 0;
  for (int xx = 0; xx < nx; ++xx) {
    const int n_kt = xx < n_ktiles ? (n_ktiles - 1 - xx) / nx + 1 : 0;
    bad |= tickets[xx] < n_kt * nkv;
  }
  const size_t head_elems = (size_t)S * D;
  const size_t n4 = (size_t)hc * head_elems / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    const size_t e0 = i * 4;
    const int h = (int)(e0 / head_elems);
    const size_t in_head = e0 - (size_t)h * head_elems;
    const int r = (int)(in_head / D);
    const int c = (int)(in_head % D);
    floatx4 acc = floatx4{};
    for (int xx = 0; xx < nx && xx < n_ktiles; ++xx) {
      if (causal && r < xx * BKV) continue;
      acc += *reinterpret_cast<const floatx4*>(partial + ((size_t)xx * hc + h) * head_elems + in_head);
    }
    floatx4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = bad ? __builtin_nanf("") : acc[e] * scale;
    *reinterpret_cast<bf16x4*>(dq + (size_t)r * tok_stride + (size_t)h * D + c) = to_out4(o, bf16());
  }
}

// Zero n ints (the queue counters, progress words and error flag).
__global__ __launch_bounds__(256) void zero_ints_kernel(int* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace upipe
