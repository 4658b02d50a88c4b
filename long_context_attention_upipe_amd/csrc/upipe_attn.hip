// Host runtime and C ABI of the UPipe attention library (declared in
// include/upipe_attn.h): argument validation, the head-chunk planner, the
// layout of the fixed buffer pool, and the per-chunk launch sequence.
//
// UPipe ("Road to 5 Million Tokens" talk summary, Chapters: heads processed
// in batches; talk digest, Quiz answer on U-Pipe): one group of heads already
// fills the GPU, so the GPU's heads run as sequential chunks and every chunk
// reuses the buffers the previous chunk used. Here the buffers are one
// caller-provided workspace carved at fixed offsets; nothing is allocated
// inside the chunk loop, and peak memory depends on head_chunk, not on Hq.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/upipe_attn.h"
#include <type_traits>

#include "attn_bf16.hpp"
#include "attn_bwd.hpp"
#include "attn_bwd_fused.hpp"
#include "attn_fwd.hpp"
#include "copy_kernels.hpp"
#include "gemm_bf16.hpp"
#include "loss_kernels.hpp"
#include "mlp_kernels.hpp"

namespace upipe {
namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Problem {
  int64_t S;
  int Hq, Hkv, d, hc, causal, dtype;
  int G;             // q heads per kv head
  int heads_per_kv;  // q heads of one chunk that share a kv head = min(hc, G)
  int nkv;           // kv heads one chunk reads = max(1, hc / G)
  size_t es;         // element size
  const int32_t* doc_off = nullptr;  // packed-document offsets (device), or null
  int n_docs = 0;
};

int validate(int64_t S, int Hq, int Hkv, int d, int hc, int causal, int dtype, Problem* pr) {
  if (S < 1) return fail(UPIPE_EINVAL, "S must be >= 1 (got %lld)", (long long)S);
  if (Hq < 1 || Hkv < 1) return fail(UPIPE_EINVAL, "Hq and Hkv must be >= 1 (got %d, %d)", Hq, Hkv);
  if (Hq % Hkv) return fail(UPIPE_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (hc < 1 || Hq % hc) return fail(UPIPE_EINVAL, "head_chunk (%d) must divide Hq (%d)", hc, Hq);
  const int G = Hq / Hkv;
  if (!(G % hc == 0 || hc % G == 0))
    return fail(UPIPE_EINVAL, "head_chunk (%d) must divide or be a multiple of Hq/Hkv (%d)", hc, G);
  if (causal != 0 && causal != 1) return fail(UPIPE_EINVAL, "causal must be 0 or 1 (got %d)", causal);
  if (dtype != UPIPE_BF16 && dtype != UPIPE_FP32) return fail(UPIPE_EUNSUPPORTED, "unsupported dtype %d", dtype);
  if (d != 64 && d != 128) return fail(UPIPE_EUNSUPPORTED, "unsupported head dim %d (64 or 128)", d);
  const size_t es = dtype == UPIPE_BF16 ? 2 : 4;
  if ((uint64_t)S * (uint64_t)d >= (1ull << 31))
    return fail(UPIPE_EUNSUPPORTED, "S*d must be < 2^31 (S=%lld, d=%d)", (long long)S, d);
  // Copy kernels index tokens with 64 bits; this only keeps byte sizes far
  // from size_t overflow (2^48 bytes = 256 TiB per tensor).
  if ((uint64_t)S * (uint64_t)std::max(Hq, Hkv) * (uint64_t)d * es >= (1ull << 48))
    return fail(UPIPE_EUNSUPPORTED, "tensor larger than 2^48 bytes");
  pr->S = S;
  pr->Hq = Hq;
  pr->Hkv = Hkv;
  pr->d = d;
  pr->hc = hc;
  pr->causal = causal;
  pr->dtype = dtype;
  pr->G = G;
  pr->heads_per_kv = std::min(hc, G);
  pr->nkv = std::max(1, hc / G);
  pr->es = es;
  return UPIPE_OK;
}

struct Chunk {
  int q_head0, kv_head0, n_kv;
  bool load_kv, first_for_kv, last_for_kv;
};

// Chunks in ascending head order. A chunk reads the kv heads of its query
// heads; when head_chunk < G several chunks share one kv head, which is then
// loaded once and its dK/dV summed over those chunks.
std::vector<Chunk> plan(const Problem& pr) {
  std::vector<Chunk> out;
  int prev_kv = -1;
  for (int h0 = 0; h0 < pr.Hq; h0 += pr.hc) {
    Chunk c;
    c.q_head0 = h0;
    c.kv_head0 = h0 / pr.G;
    c.n_kv = pr.nkv;
    c.load_kv = c.kv_head0 != prev_kv;
    c.first_for_kv = (h0 % pr.G) == 0;
    c.last_for_kv = ((h0 + pr.hc) % pr.G) == 0 || pr.hc >= pr.G;
    prev_kv = c.kv_head0;
    out.push_back(c);
  }
  return out;
}

// Pool layouts. Every chunk overwrites the same offsets.
struct FwdPool {
  size_t q, o, k, v, total;
};
// The forward's V: bf16 heads are stored transposed in blocks of 64 keys,
// [Sp/64][D][64] with Sp = S rounded up to 64 (pack_vt_kernel); fp32 heads as
// [S][D].
int64_t vt_len(const Problem& pr) { return (pr.S + 63) / 64 * 64; }
size_t vt_bytes(const Problem& pr) {
  return pr.dtype == UPIPE_BF16 ? (size_t)vt_len(pr) * pr.d * pr.es : (size_t)pr.S * pr.d * pr.es;
}
FwdPool fwd_pool(const Problem& pr) {
  const size_t U = (size_t)pr.S * pr.d * pr.es;  // one head, whole sequence
  FwdPool p;
  size_t off = 0;
  p.q = off; off += align_up(pr.hc * U);
  p.o = off; off += align_up(pr.hc * U);
  p.k = off; off += align_up(pr.nkv * U);
  p.v = off; off += align_up(pr.nkv * vt_bytes(pr));
  p.total = off;
  return p;
}

struct BwdPool {
  size_t q, dout, dq, k, v, neg_d, lse2, dk_acc, dv_acc, total;
  bool has_acc;
};
BwdPool bwd_pool(const Problem& pr) {
  const size_t U = (size_t)pr.S * pr.d * pr.es;
  BwdPool p;
  size_t off = 0;
  p.q = off; off += align_up(pr.hc * U);
  p.dout = off; off += align_up(pr.hc * U);
  p.dq = off; off += align_up(pr.hc * U);
  p.k = off; off += align_up(pr.nkv * U);
  p.v = off; off += align_up(pr.nkv * U);
  p.neg_d = off; off += align_up((size_t)pr.hc * pr.S * 4);
  p.lse2 = off; off += align_up((size_t)pr.hc * pr.S * 4);
  p.has_acc = pr.hc < pr.G;
  const size_t A = (size_t)pr.S * pr.d * 4;
  p.dk_acc = off; off += p.has_acc ? align_up(A) : 0;
  p.dv_acc = off; off += p.has_acc ? align_up(A) : 0;
  p.total = off;
  return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Grid extents of the attention kernels: the bf16 kernels' tiles for bf16,
// the generic kernels' shapes for fp32.
template <typename T, int D>
struct Tiles {
  static constexpr bool kBf16 = std::is_same<T, bf16>::value;
  static constexpr int fwd_rows = kBf16 ? Bf16Tiles::kFwdRows : FwdShape<T, D>::BQ;
  static constexpr int dq_rows = kBf16 ? Bf16Tiles::kDqRows : DqShape<T, D>::BQ;
  static constexpr int dkv_keys = kBf16 ? Bf16Tiles::kDkvKeys : DkvShape<T, D>::BKV;
};

// ---------------------------------------------------------------------------
// Optional per-kernel timing with HIP events on the launch stream.
// ---------------------------------------------------------------------------
enum KernelId {
  K_PACK = 0, K_UNPACK, K_FWD, K_BWD_PRE, K_BWD_DKDV, K_BWD_DQ, K_GEMM, K_CE_ROWS, K_SWIGLU, K_BWD_FUSED, K_DQ_REDUCE,
  K_COUNT
};
const char* const kKernelNames[K_COUNT] = {"pack_heads", "unpack_heads", "attn_fwd", "bwd_pre", "attn_bwd_dkdv",
                                           "attn_bwd_dq", "gemm_bf16", "ce_rows", "swiglu", "attn_bwd_fused",
                                           "fused_dq_reduce"};
struct Profiler {
  std::atomic<bool> on{false};
  struct Rec {
    int id;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  int64_t launches[K_COUNT] = {};
  double ms[K_COUNT] = {};
};
Profiler g_prof;
std::mutex g_prof_mu;  // guards g_prof: launches and profile calls may come from several threads

// Launch `fn` on stream `st`, bracketed by events when profiling is on.
template <typename Fn>
void timed(int id, hipStream_t st, Fn&& fn) {
  if (!g_prof.on) {
    fn();
    return;
  }
  Profiler::Rec r;
  r.id = id;
  if (hipEventCreate(&r.a) != hipSuccess) {
    fn();
    return;
  }
  if (hipEventCreate(&r.b) != hipSuccess) {
    (void)hipEventDestroy(r.a);
    fn();
    return;
  }
  const bool ok_a = hipEventRecord(r.a, st) == hipSuccess;
  fn();
  const bool ok_b = hipEventRecord(r.b, st) == hipSuccess;
  if (ok_a && ok_b) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof.pending.push_back(r);
  } else {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
}

// Caller holds g_prof_mu.
int profile_flush() {
  for (Profiler::Rec& r : g_prof.pending) {
    hipError_t e = hipEventSynchronize(r.b);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
    if (e != hipSuccess) {
      g_prof.pending.clear();
      return fail(UPIPE_EHIP, "profile: %s", hipGetErrorString(e));
    }
    g_prof.launches[r.id] += 1;
    g_prof.ms[r.id] += t;
  }
  g_prof.pending.clear();
  return UPIPE_OK;
}

unsigned copy_grid(size_t vectors) {
  const size_t blocks = (vectors + 255) / 256;
  return (unsigned)std::min<size_t>(std::max<size_t>(blocks, 1), 256 * 32);
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(UPIPE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return UPIPE_OK;
}

// The bf16 forward: the two-group kernel (256 rows per workgroup) at d = 128,
// the 4-wave kernel (128 rows) at d = 64. Sets fp.n_qtiles for the kernel.
template <int D>
void launch_attn_fwd_bf16(FwdParams<bf16> fp, hipStream_t st) {
  if constexpr (D == 128) {
    fp.n_qtiles = (fp.S + Bf16Tiles::kFwdPpRows - 1) / Bf16Tiles::kFwdPpRows;
    hipLaunchKernelGGL((attn_fwd_bf16_pp_kernel<D>), dim3(fp.n_qtiles * fp.hc), dim3(512), 0, st, fp);
  } else {
    fp.n_qtiles = (fp.S + Bf16Tiles::kFwdRows - 1) / Bf16Tiles::kFwdRows;
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D>), dim3(fp.n_qtiles * fp.hc), dim3(256), 0, st, fp);
  }
}

// The bf16 dQ kernel: the two-group kernel (256 rows per workgroup) at
// d = 128, the 4-wave kernel (128 rows) at d = 64. Sets bp.n_qtiles for it.
template <int D>
void launch_attn_dq_bf16(BwdParams<bf16> bp, hipStream_t st) {
  if constexpr (D == 128) {
    bp.n_qtiles = (bp.S + Bf16Tiles::kDqPpRows - 1) / Bf16Tiles::kDqPpRows;
    hipLaunchKernelGGL((attn_bwd_dq_bf16_pp_kernel<D>), dim3(bp.n_qtiles * bp.hc), dim3(512), 0, st, bp);
  } else {
    bp.n_qtiles = (bp.S + Bf16Tiles::kDqRows - 1) / Bf16Tiles::kDqRows;
    hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D>), dim3(bp.n_qtiles * bp.hc), dim3(256), 0, st, bp);
  }
}

template <typename T, int D>
int run_fwd(const Problem& pr, const void* q, const void* k, const void* v, void* out, void* out_lo, float* lse,
            char* ws, hipStream_t st) {
  const FwdPool pool = fwd_pool(pr);
  const int S = (int)pr.S;
  const int vpr = D * (int)sizeof(T) / 16;
  T* Qc = reinterpret_cast<T*>(ws + pool.q);
  T* Oc = reinterpret_cast<T*>(ws + pool.o);
  T* Kc = reinterpret_cast<T*>(ws + pool.k);
  T* Vc = reinterpret_cast<T*>(ws + pool.v);
  const int n_qtiles = (S + Tiles<T, D>::fwd_rows - 1) / Tiles<T, D>::fwd_rows;
  const float scale = 1.0f / std::sqrt((float)D);
  for (const Chunk& c : plan(pr)) {
    if (c.load_kv) {
      const size_t nv = (size_t)S * c.n_kv * vpr;
      timed(K_PACK, st, [&] {
        hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nv)), dim3(256), 0, st, (const uint4*)k, (uint4*)Kc, S,
                           pr.Hkv, c.kv_head0, c.n_kv, vpr);
      });
      timed(K_PACK, st, [&] {
        if constexpr (std::is_same<T, bf16>::value)
          hipLaunchKernelGGL((pack_vt_kernel<D>), dim3((unsigned)(vt_len(pr) / 64), c.n_kv), dim3(256), 0, st,
                             (const bf16*)v, (bf16*)Vc, S, (int)vt_len(pr), pr.Hkv, c.kv_head0);
        else
          hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nv)), dim3(256), 0, st, (const uint4*)v, (uint4*)Vc,
                             S, pr.Hkv, c.kv_head0, c.n_kv, vpr);
      });
    }
    const size_t nq = (size_t)S * pr.hc * vpr;
    timed(K_PACK, st, [&] {
      hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nq)), dim3(256), 0, st, (const uint4*)q, (uint4*)Qc, S,
                         pr.Hq, c.q_head0, pr.hc, vpr);
    });
    FwdParams<T> fp;
    fp.Sp = (int)vt_len(pr);
    fp.q = Qc;
    fp.k = Kc;
    fp.v = Vc;
    fp.o = Oc;
    fp.o_lo = out_lo ? reinterpret_cast<T*>(out_lo) + (size_t)c.q_head0 * D : nullptr;
    fp.H = pr.Hq;
    fp.lse = lse + (size_t)c.q_head0 * S;
    fp.S = S;
    fp.hc = pr.hc;
    fp.heads_per_kv = pr.heads_per_kv;
    fp.n_qtiles = n_qtiles;
    fp.causal = pr.causal;
    fp.doc_off = pr.doc_off;
    fp.n_docs = pr.n_docs;
    fp.scale_log2 = scale * kLog2e;
    timed(K_FWD, st, [&] {
      if constexpr (std::is_same<T, bf16>::value)
        launch_attn_fwd_bf16<D>(fp, st);
      else
        hipLaunchKernelGGL((attn_fwd_kernel<T, D>), dim3(n_qtiles * pr.hc), dim3(256), 0, st, fp);
    });
    timed(K_UNPACK, st, [&] {
      hipLaunchKernelGGL(unpack_heads_kernel, dim3(copy_grid(nq)), dim3(256), 0, st, (const uint4*)Oc, (uint4*)out, S,
                         pr.Hq, c.q_head0, pr.hc, vpr);
    });
    if (int rc = check_launch("forward chunk")) return rc;
  }
  return UPIPE_OK;
}

template <typename T, int D>
int run_bwd(const Problem& pr, const void* q, const void* k, const void* v, const void* out, const void* out_lo,
            const void* dout, const float* lse, void* dq, void* dk, void* dv, char* ws, hipStream_t st) {
  const BwdPool pool = bwd_pool(pr);
  const int S = (int)pr.S;
  const int vpr = D * (int)sizeof(T) / 16;
  T* Qc = reinterpret_cast<T*>(ws + pool.q);
  T* dOc = reinterpret_cast<T*>(ws + pool.dout);
  T* dQc = reinterpret_cast<T*>(ws + pool.dq);
  T* Kc = reinterpret_cast<T*>(ws + pool.k);
  T* Vc = reinterpret_cast<T*>(ws + pool.v);
  float* nDc = reinterpret_cast<float*>(ws + pool.neg_d);
  float* L2c = reinterpret_cast<float*>(ws + pool.lse2);
  float* dKa = pool.has_acc ? reinterpret_cast<float*>(ws + pool.dk_acc) : nullptr;
  float* dVa = pool.has_acc ? reinterpret_cast<float*>(ws + pool.dv_acc) : nullptr;
  const int n_qtiles = (S + Tiles<T, D>::dq_rows - 1) / Tiles<T, D>::dq_rows;
  const int n_ktiles = (S + Tiles<T, D>::dkv_keys - 1) / Tiles<T, D>::dkv_keys;
  const float scale = 1.0f / std::sqrt((float)D);
  constexpr int kRowsPerPreBlock = 256 / (D * (int)sizeof(T) / 16);
  for (const Chunk& c : plan(pr)) {
    if (c.load_kv) {
      const size_t nv = (size_t)S * c.n_kv * vpr;
      timed(K_PACK, st, [&] {
        hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nv)), dim3(256), 0, st, (const uint4*)k, (uint4*)Kc, S,
                           pr.Hkv, c.kv_head0, c.n_kv, vpr);
      });
      timed(K_PACK, st, [&] {
        hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nv)), dim3(256), 0, st, (const uint4*)v, (uint4*)Vc, S,
                           pr.Hkv, c.kv_head0, c.n_kv, vpr);
      });
    }
    const size_t nq = (size_t)S * pr.hc * vpr;
    timed(K_PACK, st, [&] {
      hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nq)), dim3(256), 0, st, (const uint4*)q, (uint4*)Qc, S,
                         pr.Hq, c.q_head0, pr.hc, vpr);
    });
    const size_t rows = (size_t)S * pr.hc;
    const unsigned pre_grid =
        (unsigned)std::min<size_t>((rows + kRowsPerPreBlock - 1) / kRowsPerPreBlock, 256 * 32);
    timed(K_BWD_PRE, st, [&] {
      const int64_t tok = (int64_t)pr.Hq * D, h0 = (int64_t)c.q_head0 * D;  // caller's [S, Hq, d]
      const RowsView<T> o_v{reinterpret_cast<const T*>(out) + h0, tok, D};
      const RowsView<T> lo_v{out_lo ? reinterpret_cast<const T*>(out_lo) + h0 : nullptr, tok, D};
      const RowsView<T> do_v{reinterpret_cast<const T*>(dout) + h0, tok, D};
      hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(pre_grid), dim3(256), 0, st, o_v, lo_v, do_v,
                         lse + (size_t)c.q_head0 * S, dOc, nDc, L2c, S, pr.hc);
    });

    BwdParams<T> bp;
    bp.q = Qc;
    bp.k = Kc;
    bp.v = Vc;
    bp.dout = dOc;
    bp.lse = lse + (size_t)c.q_head0 * S;
    bp.negD = nDc;
    bp.lse2 = L2c;
    bp.dq = dQc;
    bp.dk_acc = dKa;
    bp.dv_acc = dVa;
    bp.dk_out = reinterpret_cast<T*>(dk) + (size_t)c.kv_head0 * D;
    bp.dv_out = reinterpret_cast<T*>(dv) + (size_t)c.kv_head0 * D;
    bp.Hkv_total = pr.Hkv;
    bp.S = S;
    bp.hc = pr.hc;
    bp.heads_per_kv = pr.heads_per_kv;
    bp.nkv = pr.nkv;
    bp.n_qtiles = n_qtiles;
    bp.n_ktiles = n_ktiles;
    bp.causal = pr.causal;
    bp.doc_off = pr.doc_off;
    bp.n_docs = pr.n_docs;
    bp.acc_load = !c.first_for_kv;
    bp.finalize = c.last_for_kv;
    bp.scale = scale;
    bp.scale_log2 = scale * kLog2e;
    timed(K_BWD_DKDV, st, [&] {
      if constexpr (std::is_same<T, bf16>::value)
        hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D>), dim3(n_ktiles * pr.nkv), dim3(256), 0, st, bp);
      else
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D>), dim3(n_ktiles * pr.nkv), dim3(256), 0, st, bp);
    });
    timed(K_BWD_DQ, st, [&] {
      if constexpr (std::is_same<T, bf16>::value)
        launch_attn_dq_bf16<D>(bp, st);
      else
        hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D>), dim3(n_qtiles * pr.hc), dim3(256), 0, st, bp);
    });
    timed(K_UNPACK, st, [&] {
      hipLaunchKernelGGL(unpack_heads_kernel, dim3(copy_grid(nq)), dim3(256), 0, st, (const uint4*)dQc, (uint4*)dq, S,
                         pr.Hq, c.q_head0, pr.hc, vpr);
    });
    if (int rc = check_launch("backward chunk")) return rc;
  }
  return UPIPE_OK;
}

// ---------------------------------------------------------------------------
// The fused deterministic backward (attn_bwd_fused.hpp): bf16, d = 128, no
// document masks. Pool: the two-kernel backward's buffers without its packed
// dQ, plus one fp32 dQ partial per XCD and the queue/progress words.
// ---------------------------------------------------------------------------
constexpr int kMaxXcd = 8;
constexpr int kDefaultMaxPolls = 1 << 20;

struct FusedPool {
  size_t q, dout, k, v, neg_d, lse2, dk_acc, dv_acc, partial, sync, total;
  size_t sync_ints;  // tickets [kMaxXcd], error [1], progress [n_ktiles][nkv][4]
  bool has_acc;
};
FusedPool fused_pool(const Problem& pr) {
  const size_t U = (size_t)pr.S * pr.d * pr.es;
  const int64_t n_ktiles = (pr.S + Bf16Tiles::kDkvKeys - 1) / Bf16Tiles::kDkvKeys;
  FusedPool p;
  size_t off = 0;
  p.q = off; off += align_up(pr.hc * U);
  p.dout = off; off += align_up(pr.hc * U);
  p.k = off; off += align_up(pr.nkv * U);
  p.v = off; off += align_up(pr.nkv * U);
  p.neg_d = off; off += align_up((size_t)pr.hc * pr.S * 4);
  p.lse2 = off; off += align_up((size_t)pr.hc * pr.S * 4);
  p.has_acc = pr.hc < pr.G;
  const size_t A = (size_t)pr.S * pr.d * 4;
  p.dk_acc = off; off += p.has_acc ? align_up(A) : 0;
  p.dv_acc = off; off += p.has_acc ? align_up(A) : 0;
  p.partial = off; off += align_up((size_t)kMaxXcd * pr.hc * A);
  p.sync_ints = kMaxXcd + 1 + (size_t)n_ktiles * pr.nkv * 4;
  p.sync = off; off += align_up(p.sync_ints * 4);
  p.total = off;
  return p;
}

// The fused path's limits on top of validate(): bf16 heads of 128, and the
// per-XCD partial of one head addressed with 32-bit byte offsets.
int validate_fused(const Problem& pr) {
  if (pr.dtype != UPIPE_BF16) return fail(UPIPE_EUNSUPPORTED, "the fused backward supports bf16 only");
  if (pr.d != 128) return fail(UPIPE_EUNSUPPORTED, "the fused backward supports d = 128 only (got %d)", pr.d);
  if ((uint64_t)(pr.S + Bf16Tiles::kDkvRows) * 128 * 4 > 0xFFFFFFFFull)
    return fail(UPIPE_EUNSUPPORTED, "the fused backward needs (S + 32) * 512 < 2^32 (S = %lld)", (long long)pr.S);
  return UPIPE_OK;
}

// XCD count and resident-workgroup capacity of the current device, looked up
// once per device.
struct DeviceShape {
  int nx = 0, cus = 0;
};
std::mutex g_shape_mu;
std::vector<DeviceShape> g_shapes;

int device_shape(DeviceShape* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(UPIPE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_shape_mu);
  if ((int)g_shapes.size() <= dev) g_shapes.resize(dev + 1);
  DeviceShape& d = g_shapes[dev];
  if (!d.nx) {
    int nx = 0, cus = 0;
    e = hipDeviceGetAttribute(&nx, hipDeviceAttributeNumberOfXccs, dev);
    if (e != hipSuccess) return fail(UPIPE_EHIP, "XCD count of device %d: %s", dev, hipGetErrorString(e));
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(UPIPE_EHIP, "CU count of device %d: %s", dev, hipGetErrorString(e));
    if (nx < 1 || nx > kMaxXcd) return fail(UPIPE_EUNSUPPORTED, "device %d reports %d XCDs (1..%d)", dev, nx, kMaxXcd);
    d.nx = nx;
    d.cus = std::max(cus, nx);
  }
  *out = d;
  return UPIPE_OK;
}

template <int D>
int run_bwd_fused(const Problem& pr, const void* q, const void* k, const void* v, const void* out,
                  const void* out_lo, const void* dout, const float* lse, void* dq, void* dk, void* dv, char* ws,
                  int max_polls, hipStream_t st) {
  static_assert(D == 128, "the fused kernel is written for d = 128");
  DeviceShape dsh;
  if (int rc = device_shape(&dsh)) return rc;
  const FusedPool pool = fused_pool(pr);
  const int S = (int)pr.S;
  const int vpr = D * 2 / 16;
  bf16* Qc = reinterpret_cast<bf16*>(ws + pool.q);
  bf16* dOc = reinterpret_cast<bf16*>(ws + pool.dout);
  bf16* Kc = reinterpret_cast<bf16*>(ws + pool.k);
  bf16* Vc = reinterpret_cast<bf16*>(ws + pool.v);
  float* nDc = reinterpret_cast<float*>(ws + pool.neg_d);
  float* L2c = reinterpret_cast<float*>(ws + pool.lse2);
  float* dKa = pool.has_acc ? reinterpret_cast<float*>(ws + pool.dk_acc) : nullptr;
  float* dVa = pool.has_acc ? reinterpret_cast<float*>(ws + pool.dv_acc) : nullptr;
  int* sync = reinterpret_cast<int*>(ws + pool.sync);
  const int n_ktiles = (S + Bf16Tiles::kDkvKeys - 1) / Bf16Tiles::kDkvKeys;
  const float scale = 1.0f / std::sqrt((float)D);
  constexpr int kRowsPerPreBlock = 256 / (D * 2 / 16);
  // Resident capacity (two workgroups per CU), at least one workgroup per
  // XCD; workgroups past the tiles of their XCD's queue leave at once.
  const int n_tiles = n_ktiles * pr.nkv;
  const unsigned grid = (unsigned)std::max(std::min(2 * dsh.cus, n_tiles), dsh.nx);
  for (const Chunk& c : plan(pr)) {
    if (c.load_kv) {
      const size_t nv = (size_t)S * c.n_kv * vpr;
      timed(K_PACK, st, [&] {
        hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nv)), dim3(256), 0, st, (const uint4*)k, (uint4*)Kc, S,
                           pr.Hkv, c.kv_head0, c.n_kv, vpr);
      });
      timed(K_PACK, st, [&] {
        hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nv)), dim3(256), 0, st, (const uint4*)v, (uint4*)Vc, S,
                           pr.Hkv, c.kv_head0, c.n_kv, vpr);
      });
    }
    const size_t nq = (size_t)S * pr.hc * vpr;
    timed(K_PACK, st, [&] {
      hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nq)), dim3(256), 0, st, (const uint4*)q, (uint4*)Qc, S,
                         pr.Hq, c.q_head0, pr.hc, vpr);
    });
    const size_t rows = (size_t)S * pr.hc;
    const unsigned pre_grid =
        (unsigned)std::min<size_t>((rows + kRowsPerPreBlock - 1) / kRowsPerPreBlock, 256 * 32);
    timed(K_BWD_PRE, st, [&] {
      const int64_t tok = (int64_t)pr.Hq * D, h0 = (int64_t)c.q_head0 * D;
      const RowsView<bf16> o_v{reinterpret_cast<const bf16*>(out) + h0, tok, D};
      const RowsView<bf16> lo_v{out_lo ? reinterpret_cast<const bf16*>(out_lo) + h0 : nullptr, tok, D};
      const RowsView<bf16> do_v{reinterpret_cast<const bf16*>(dout) + h0, tok, D};
      hipLaunchKernelGGL((bwd_pre_kernel<bf16, D>), dim3(pre_grid), dim3(256), 0, st, o_v, lo_v, do_v,
                         lse + (size_t)c.q_head0 * S, dOc, nDc, L2c, S, pr.hc);
    });
    hipLaunchKernelGGL(zero_ints_kernel, dim3(copy_grid(pool.sync_ints)), dim3(256), 0, st, sync, pool.sync_ints);

    BwdParams<bf16> bp = {};
    bp.q = Qc;
    bp.k = Kc;
    bp.v = Vc;
    bp.dout = dOc;
    bp.lse = lse + (size_t)c.q_head0 * S;
    bp.negD = nDc;
    bp.lse2 = L2c;
    bp.dq = nullptr;
    bp.dk_acc = dKa;
    bp.dv_acc = dVa;
    bp.dk_out = reinterpret_cast<bf16*>(dk) + (size_t)c.kv_head0 * D;
    bp.dv_out = reinterpret_cast<bf16*>(dv) + (size_t)c.kv_head0 * D;
    bp.Hkv_total = pr.Hkv;
    bp.S = S;
    bp.hc = pr.hc;
    bp.heads_per_kv = pr.heads_per_kv;
    bp.nkv = pr.nkv;
    bp.n_ktiles = n_ktiles;
    bp.causal = pr.causal;
    bp.acc_load = !c.first_for_kv;
    bp.finalize = c.last_for_kv;
    bp.scale = scale;
    bp.scale_log2 = scale * kLog2e;
    FusedSync fs;
    fs.partial = reinterpret_cast<float*>(ws + pool.partial);
    fs.tickets = sync;
    fs.error = sync + kMaxXcd;
    fs.progress = sync + kMaxXcd + 1;
    fs.nx = dsh.nx;
    fs.max_polls = max_polls;
    timed(K_BWD_FUSED, st, [&] {
      hipLaunchKernelGGL((attn_bwd_fused_bf16_kernel<D>), dim3(grid), dim3(256), 0, st, bp, fs);
    });
    timed(K_DQ_REDUCE, st, [&] {
      const size_t n4 = (size_t)pr.hc * S * D / 4;
      hipLaunchKernelGGL(fused_dq_reduce_kernel, dim3(copy_grid(n4)), dim3(256), 0, st, fs.partial, fs.tickets,
                         fs.error, reinterpret_cast<bf16*>(dq) + (size_t)c.q_head0 * D, (int64_t)pr.Hq * D, S, pr.hc,
                         dsh.nx, n_ktiles, pr.nkv, pr.causal, scale);
    });
    if (int rc = check_launch("fused backward chunk")) return rc;
  }
  return UPIPE_OK;
}

// ---------------------------------------------------------------------------
// bf16 GEMM (gemm_bf16.hpp): argument checks and launch.
// ---------------------------------------------------------------------------
constexpr int64_t kUnblocked = (int64_t)1 << 62;  // a contiguous index that never wraps

// log2 of a block length that is a power of two >= 8, else -1.
int block_shift(int64_t blk) {
  if (blk < 8 || (blk & (blk - 1))) return -1;
  int sh = 0;
  while ((int64_t(1) << sh) < blk) ++sh;
  return sh;
}

GemmOperand operand(const void* p, int64_t ld, int kmajor, int64_t blk = kUnblocked, int64_t blk_stride = 0,
                    int kvalid = 1 << 30) {
  GemmOperand o;
  o.p = reinterpret_cast<const bf16*>(p);
  o.ld = ld;
  o.blk_shift = block_shift(blk);
  o.blk_stride = blk_stride;
  o.kmajor = kmajor;
  o.kvalid = kvalid;
  return o;
}

template <typename CT>
GemmOut<CT> gemm_out(CT* p, int64_t ldc, int64_t blk = kUnblocked, int64_t blk_stride = 0) {
  return GemmOut<CT>{p, ldc, block_shift(blk), blk_stride};
}

int check_operand(const char* name, const GemmOperand& o, int MN, int K) {
  if (!o.p) return fail(UPIPE_EINVAL, "%s is NULL", name);
  if ((uintptr_t)o.p % 16) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", name);
  if (o.ld < 1 || o.ld % 8) return fail(UPIPE_EINVAL, "%s: leading dimension %lld is not a positive multiple of 8",
                                        name, (long long)o.ld);
  if (o.blk_shift < 3 || (o.blk_shift < 62 && (o.blk_stride < 0 || o.blk_stride % 8)))
    return fail(UPIPE_EINVAL, "%s: block length must be a power of two >= 8 and the block stride a multiple of 8",
                name);
  if (!o.kmajor && MN % 8) return fail(UPIPE_EINVAL, "%s: an M/N-contiguous operand needs M or N a multiple of 8", name);
  (void)K;
  return UPIPE_OK;
}

template <typename CT>
int gemm(const GemmOperand& a, const GemmOperand& b, const GemmOut<CT>& c, int M, int N, int K, int accumulate,
         hipStream_t st) {
  GemmParams<CT> p;
  p.a = a;
  p.b = b;
  p.c = c;
  p.M = M;
  p.N = N;
  p.K = K;
  p.accumulate = accumulate;
  p.k_split = 0;
  p.partial = nullptr;
  // 256 x 256 tiles (one 8-wave workgroup per CU) when there is at least one
  // per CU; 128 x 128 tiles (two 4-wave workgroups per CU) otherwise.
  const int64_t big_tiles = ((int64_t)M + 255) / 256 * (((int64_t)N + 255) / 256);
  if (big_tiles >= 256) {
    const dim3 grid((unsigned)((M + 255) / 256), (unsigned)((N + 255) / 256));
    if (a.kmajor && b.kmajor)
      hipLaunchKernelGGL((gemm_bf16_256_kernel<CT, 1, 1>), grid, dim3(512), 0, st, p);
    else if (a.kmajor)
      hipLaunchKernelGGL((gemm_bf16_256_kernel<CT, 1, 0>), grid, dim3(512), 0, st, p);
    else if (b.kmajor)
      hipLaunchKernelGGL((gemm_bf16_256_kernel<CT, 0, 1>), grid, dim3(512), 0, st, p);
    else
      hipLaunchKernelGGL((gemm_bf16_256_kernel<CT, 0, 0>), grid, dim3(512), 0, st, p);
    return check_launch("gemm");
  }
  const dim3 grid((unsigned)((M + 127) / 128), (unsigned)((N + 127) / 128));
  if (a.kmajor && b.kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<CT, 1, 1>), grid, dim3(256), 0, st, p);
  else if (a.kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<CT, 1, 0>), grid, dim3(256), 0, st, p);
  else if (b.kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<CT, 0, 1>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<CT, 0, 0>), grid, dim3(256), 0, st, p);
  return check_launch("gemm");
}

// The same product with K split into ranges of k_split (a multiple of 64):
// one workgroup per (128 x 128 tile, range) writes its fp32 partial product
// to `partial` ([ranges][M][N]), and a second kernel adds the ranges in
// ascending order into C (C += when accumulate). For products with few tiles
// and a long K (the weight gradients, contracted over every token).
template <typename CT>
int gemm_split(const GemmOperand& a, const GemmOperand& b, const GemmOut<CT>& c, int M, int N, int K, int k_split,
               int accumulate, float* partial, hipStream_t st) {
  GemmParams<CT> p;
  p.a = a;
  p.b = b;
  p.c = c;
  p.M = M;
  p.N = N;
  p.K = K;
  p.accumulate = 0;
  p.k_split = k_split;
  p.partial = partial;
  const int n_split = (K + k_split - 1) / k_split;
  const dim3 grid((unsigned)((M + 127) / 128), (unsigned)((N + 127) / 128), (unsigned)n_split);
  if (a.kmajor && b.kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<CT, 1, 1>), grid, dim3(256), 0, st, p);
  else if (a.kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<CT, 1, 0>), grid, dim3(256), 0, st, p);
  else if (b.kmajor)
    hipLaunchKernelGGL((gemm_bf16_kernel<CT, 0, 1>), grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<CT, 0, 0>), grid, dim3(256), 0, st, p);
  hipLaunchKernelGGL((gemm_split_reduce_kernel<CT>), dim3(copy_grid((size_t)M * N / 4)), dim3(256), 0, st, partial,
                     n_split, M, N, c, accumulate);
  return check_launch("split gemm");
}

// How the token-contracting products split their K = S rows (whole 64-row
// steps): up to 64 ranges of at least 8192 tokens, a function of S alone, so
// every head_chunk adds each weight gradient's terms in the same order.
struct TokenSplit {
  int k_split, n_split;  // n_split < 2: no split
};
TokenSplit token_split(int64_t S) {
  const int64_t K0 = S / 64 * 64;
  const int64_t n = std::min<int64_t>(64, K0 / 8192);
  if (n < 2) return {0, 1};
  const int64_t k = (K0 / n + 63) / 64 * 64;
  return {(int)k, (int)((K0 + k - 1) / k)};
}

// ---------------------------------------------------------------------------
// Attention block (projections around the chunked attention), forward.
// Pool: the chunk's q and attention output rows (head-major), its kv heads'
// k rows, their v rows token-major as the projection writes them and again
// transposed for the forward kernel. Every chunk reuses the same offsets.
// ---------------------------------------------------------------------------
struct BlockPool {
  size_t q, o, k, vtmp, vt, total;
};
BlockPool block_pool(const Problem& pr) {
  const size_t U = (size_t)pr.S * pr.d * pr.es;
  BlockPool p;
  size_t off = 0;
  p.q = off; off += align_up(pr.hc * U);
  p.o = off; off += align_up(pr.hc * U);
  p.k = off; off += align_up(pr.nkv * U);
  p.vtmp = off; off += align_up(pr.nkv * U);
  p.vt = off; off += align_up(pr.nkv * vt_bytes(pr));
  p.total = off;
  return p;
}

int validate_block(int64_t S, int Dm, int Hq, int Hkv, int d, int hc, int causal, Problem* pr) {
  if (int rc = validate(S, Hq, Hkv, d, hc, causal, UPIPE_BF16, pr)) return rc;
  if (Dm < 64 || Dm % 64) return fail(UPIPE_EUNSUPPORTED, "model dim Dm (%d) must be a positive multiple of 64", Dm);
  if ((uint64_t)S * (uint64_t)Dm * 4 >= (1ull << 48)) return fail(UPIPE_EUNSUPPORTED, "x larger than 2^48 bytes");
  return UPIPE_OK;
}

template <int D>
int run_block_fwd(const Problem& pr, int Dm, const void* x, const void* wq, const void* wk, const void* wv,
                  const void* wo, float* y, void* out, float* lse, char* ws, hipStream_t st) {
  const BlockPool pool = block_pool(pr);
  const int S = (int)pr.S;
  bf16* Qc = reinterpret_cast<bf16*>(ws + pool.q);
  bf16* Oc = reinterpret_cast<bf16*>(ws + pool.o);
  bf16* Kc = reinterpret_cast<bf16*>(ws + pool.k);
  bf16* Vtmp = reinterpret_cast<bf16*>(ws + pool.vtmp);
  bf16* Vt = reinterpret_cast<bf16*>(ws + pool.vt);
  const int n_qtiles = (S + Bf16Tiles::kFwdRows - 1) / Bf16Tiles::kFwdRows;
  const float scale = 1.0f / std::sqrt((float)D);
  const int64_t SD = (int64_t)S * D;
  const GemmOperand xa = operand(x, Dm, 1);  // [S][Dm], K = Dm contiguous
  for (const Chunk& c : plan(pr)) {
    if (c.load_kv) {
      // k of the chunk's kv heads, head-major [nkv][S][D]; v token-major [S][nkv*D]
      const GemmOperand wkb = operand(reinterpret_cast<const bf16*>(wk) + (int64_t)c.kv_head0 * D * Dm, Dm, 1);
      const GemmOperand wvb = operand(reinterpret_cast<const bf16*>(wv) + (int64_t)c.kv_head0 * D * Dm, Dm, 1);
      GemmOut<bf16> kout = gemm_out(Kc, D, D, SD);
      GemmOut<bf16> vout = gemm_out(Vtmp, (int64_t)c.n_kv * D);
      timed(K_GEMM, st, [&] { (void)gemm(xa, wkb, kout, S, c.n_kv * D, Dm, 0, st); });
      timed(K_GEMM, st, [&] { (void)gemm(xa, wvb, vout, S, c.n_kv * D, Dm, 0, st); });
      timed(K_PACK, st, [&] {
        hipLaunchKernelGGL((pack_vt_kernel<D>), dim3((unsigned)(vt_len(pr) / 64), c.n_kv), dim3(256), 0, st, Vtmp,
                           Vt, S, (int)vt_len(pr), c.n_kv, 0);
      });
    }
    const GemmOperand wqb = operand(reinterpret_cast<const bf16*>(wq) + (int64_t)c.q_head0 * D * Dm, Dm, 1);
    GemmOut<bf16> qout = gemm_out(Qc, D, D, SD);
    timed(K_GEMM, st, [&] { (void)gemm(xa, wqb, qout, S, pr.hc * D, Dm, 0, st); });
    FwdParams<bf16> fp;
    fp.Sp = (int)vt_len(pr);
    fp.q = Qc;
    fp.k = Kc;
    fp.v = Vt;
    fp.o = Oc;
    fp.o_lo = nullptr;
    fp.H = pr.Hq;
    fp.lse = lse + (size_t)c.q_head0 * S;
    fp.S = S;
    fp.hc = pr.hc;
    fp.heads_per_kv = pr.heads_per_kv;
    fp.n_qtiles = n_qtiles;
    fp.causal = pr.causal;
    fp.doc_off = nullptr;
    fp.n_docs = 0;
    fp.scale_log2 = scale * kLog2e;
    timed(K_FWD, st, [&] {
      launch_attn_fwd_bf16<D>(fp, st);
    });
    if (out) {
      const size_t nq = (size_t)S * pr.hc * (D / 8);
      timed(K_UNPACK, st, [&] {
        hipLaunchKernelGGL(unpack_heads_kernel, dim3(copy_grid(nq)), dim3(256), 0, st, (const uint4*)Oc, (uint4*)out,
                           S, pr.Hq, c.q_head0, pr.hc, D / 8);
      });
    }
    // y (+)= o_h Wo_h^T one head at a time, in head order, so y's fp32 sums
    // do not depend on head_chunk
    for (int hl = 0; hl < pr.hc; ++hl) {
      const int h = c.q_head0 + hl;
      const GemmOperand oa = operand(Oc + (int64_t)hl * SD, D, 1);
      const GemmOperand wob = operand(reinterpret_cast<const bf16*>(wo) + (int64_t)h * D, (int64_t)pr.Hq * D, 1);
      GemmOut<float> yout = gemm_out(y, Dm);
      timed(K_GEMM, st, [&] { (void)gemm(oa, wob, yout, S, Dm, D, h > 0, st); });
    }
    if (int rc = check_launch("attention block chunk")) return rc;
  }
  return UPIPE_OK;
}

// ---------------------------------------------------------------------------
// Attention block, backward. Pool: the chunk's q, o, dO and dq rows
// (head-major), its kv heads' k and v rows (head-major) and their dk, dv rows
// (token-major, as the dK/dV kernel writes them), -D and lse*log2(e) rows,
// the fp32 dK/dV partials when chunks split a kv group, and the zero-padded
// last rows of x and dy; when o is recomputed, also the transposed v, o's
// rounding residual and the recomputed lse. Every chunk reuses the offsets.
// ---------------------------------------------------------------------------
struct BlockBwdPool {
  size_t q, o, dout, dq, k, v, dk, dv, neg_d, lse2, dk_acc, dv_acc, xtail, dytail, vt, olo, lrec, split, total;
  bool has_acc;
};
BlockBwdPool block_bwd_pool(const Problem& pr, int Dm, bool recompute) {
  const size_t U = (size_t)pr.S * pr.d * 2;
  const size_t R = (size_t)pr.hc * pr.S * 4;
  BlockBwdPool p;
  size_t off = 0;
  p.q = off; off += align_up(pr.hc * U);
  p.o = off; off += align_up(pr.hc * U);
  p.dout = off; off += align_up(pr.hc * U);
  p.dq = off; off += align_up(pr.hc * U);
  p.k = off; off += align_up(pr.nkv * U);
  p.v = off; off += align_up(pr.nkv * U);
  p.dk = off; off += align_up(pr.nkv * U);
  p.dv = off; off += align_up(pr.nkv * U);
  p.neg_d = off; off += align_up(R);
  p.lse2 = off; off += align_up(R);
  p.has_acc = pr.hc < pr.G;
  const size_t A = (size_t)pr.S * pr.d * 4;
  p.dk_acc = off; off += p.has_acc ? align_up(A) : 0;
  p.dv_acc = off; off += p.has_acc ? align_up(A) : 0;
  p.xtail = off; off += align_up((size_t)64 * Dm * 2);
  p.dytail = off; off += align_up((size_t)64 * Dm * 2);
  p.vt = off; off += recompute ? align_up(pr.nkv * vt_bytes(pr)) : 0;
  p.olo = off; off += recompute ? align_up(pr.hc * U) : 0;
  p.lrec = off; off += recompute ? align_up(R) : 0;
  // fp32 partial products of the split weight-gradient GEMMs (the largest is hc*d x Dm)
  const TokenSplit ts = token_split(pr.S);
  p.split = off; off += ts.n_split > 1 ? align_up((size_t)ts.n_split * pr.hc * pr.d * Dm * 4) : 0;
  p.total = off;
  return p;
}

// C (+)= A B with K = S (a contraction over tokens) for A, B given as
// [K = token][M or N] operands: the first K0 = S rounded down to 64 tokens
// directly, the last S - K0 through the zero-padded copy `b_tail` of B's last
// rows (A's rows past S are read as its last row, against those zeros).
// `a_tail` is A advanced by K0 tokens.
template <typename CT>
int gemm_over_tokens(const GemmOperand& a, const GemmOperand& a_tail, const GemmOperand& b, const GemmOperand& b_tail,
                     const GemmOut<CT>& c, int M, int N, int S, float* split_buf, hipStream_t st) {
  const int K0 = S / 64 * 64;
  const TokenSplit ts = token_split(S);
  if (K0 > 0 && ts.n_split > 1)
    timed(K_GEMM, st, [&] { (void)gemm_split(a, b, c, M, N, K0, ts.k_split, 0, split_buf, st); });
  else if (K0 > 0)
    timed(K_GEMM, st, [&] { (void)gemm(a, b, c, M, N, K0, 0, st); });
  if (S > K0) timed(K_GEMM, st, [&] { (void)gemm(a_tail, b_tail, c, M, N, 64, K0 > 0, st); });
  return check_launch("gemm over tokens");
}

template <int D>
int run_block_bwd(const Problem& pr, int Dm, const void* x, const void* wq, const void* wk, const void* wv,
                  const void* wo, const void* dy, const void* out, const float* lse, float* dx, float* dwq,
                  float* dwk, float* dwv, float* dwo, char* ws, hipStream_t st) {
  const bool recompute = out == nullptr;
  const BlockBwdPool pool = block_bwd_pool(pr, Dm, recompute);
  const int S = (int)pr.S;
  const int64_t SD = (int64_t)S * D;
  const int K0 = S / 64 * 64, tail = S - K0;
  bf16* Qc = reinterpret_cast<bf16*>(ws + pool.q);
  bf16* Oc = reinterpret_cast<bf16*>(ws + pool.o);
  bf16* dOc = reinterpret_cast<bf16*>(ws + pool.dout);
  bf16* dQc = reinterpret_cast<bf16*>(ws + pool.dq);
  bf16* Kc = reinterpret_cast<bf16*>(ws + pool.k);
  bf16* Vc = reinterpret_cast<bf16*>(ws + pool.v);
  bf16* dKc = reinterpret_cast<bf16*>(ws + pool.dk);
  bf16* dVc = reinterpret_cast<bf16*>(ws + pool.dv);
  float* nDc = reinterpret_cast<float*>(ws + pool.neg_d);
  float* L2c = reinterpret_cast<float*>(ws + pool.lse2);
  float* dKa = pool.has_acc ? reinterpret_cast<float*>(ws + pool.dk_acc) : nullptr;
  float* dVa = pool.has_acc ? reinterpret_cast<float*>(ws + pool.dv_acc) : nullptr;
  bf16* xtail = reinterpret_cast<bf16*>(ws + pool.xtail);
  bf16* dytail = reinterpret_cast<bf16*>(ws + pool.dytail);
  bf16* Vt = recompute ? reinterpret_cast<bf16*>(ws + pool.vt) : nullptr;
  bf16* OLc = recompute ? reinterpret_cast<bf16*>(ws + pool.olo) : nullptr;
  float* Lrec = recompute ? reinterpret_cast<float*>(ws + pool.lrec) : nullptr;
  float* split_buf = reinterpret_cast<float*>(ws + pool.split);
  const bf16* xb = reinterpret_cast<const bf16*>(x);
  const bf16* dyb = reinterpret_cast<const bf16*>(dy);
  const int n_fwd_tiles = (S + Bf16Tiles::kFwdRows - 1) / Bf16Tiles::kFwdRows;
  const int n_qtiles = (S + Bf16Tiles::kDqRows - 1) / Bf16Tiles::kDqRows;
  const int n_ktiles = (S + Bf16Tiles::kDkvKeys - 1) / Bf16Tiles::kDkvKeys;
  const float scale = 1.0f / std::sqrt((float)D);
  const GemmOperand xa = operand(x, Dm, 1);    // [S][Dm], K = Dm contiguous
  const GemmOperand dya = operand(dy, Dm, 1);  // the same for dy
  // x and dy as [K = token][N or M = Dm] operands, and their padded last rows
  const GemmOperand x_tok = operand(x, Dm, 0), x_tail = operand(xtail, Dm, 0);
  const GemmOperand dy_tok = operand(dy, Dm, 0), dy_tail = operand(dytail, Dm, 0);
  if (tail > 0) {
    timed(K_PACK, st, [&] {
      hipLaunchKernelGGL(tail_rows_kernel, dim3(64), dim3(256), 0, st, xb + (int64_t)K0 * Dm, xtail, tail, Dm);
    });
    timed(K_PACK, st, [&] {
      hipLaunchKernelGGL(tail_rows_kernel, dim3(64), dim3(256), 0, st, dyb + (int64_t)K0 * Dm, dytail, tail, Dm);
    });
  }
  bool dx_started = false;
  for (const Chunk& c : plan(pr)) {
    if (c.load_kv) {
      // k and v of the chunk's kv heads, head-major [nkv][S][D]
      const GemmOperand wkb = operand(reinterpret_cast<const bf16*>(wk) + (int64_t)c.kv_head0 * D * Dm, Dm, 1);
      const GemmOperand wvb = operand(reinterpret_cast<const bf16*>(wv) + (int64_t)c.kv_head0 * D * Dm, Dm, 1);
      timed(K_GEMM, st, [&] { (void)gemm(xa, wkb, gemm_out(Kc, D, D, SD), S, c.n_kv * D, Dm, 0, st); });
      timed(K_GEMM, st, [&] { (void)gemm(xa, wvb, gemm_out(Vc, D, D, SD), S, c.n_kv * D, Dm, 0, st); });
      if (recompute)
        for (int g = 0; g < c.n_kv; ++g)
          timed(K_PACK, st, [&] {
            hipLaunchKernelGGL((pack_vt_kernel<D>), dim3((unsigned)(vt_len(pr) / 64), 1), dim3(256), 0, st,
                               Vc + g * SD, Vt + (int64_t)g * D * vt_len(pr), S, (int)vt_len(pr), 1, 0);
          });
    }
    // q of the chunk's heads and dO = dy Wo (Wo's columns of those heads, as
    // [K = Dm][N = hc*D]), both head-major [hc][S][D]
    const GemmOperand wqb = operand(reinterpret_cast<const bf16*>(wq) + (int64_t)c.q_head0 * D * Dm, Dm, 1);
    timed(K_GEMM, st, [&] { (void)gemm(xa, wqb, gemm_out(Qc, D, D, SD), S, pr.hc * D, Dm, 0, st); });
    const GemmOperand wo_cols = operand(reinterpret_cast<const bf16*>(wo) + (int64_t)c.q_head0 * D, (int64_t)pr.Hq * D, 0);
    timed(K_GEMM, st, [&] { (void)gemm(dya, wo_cols, gemm_out(dOc, D, D, SD), S, pr.hc * D, Dm, 0, st); });
    // o of the chunk's heads: the caller's, or the forward run again
    RowsView<bf16> lo_v{nullptr, 0, 0};
    const float* lse_c;
    if (recompute) {
      FwdParams<bf16> fp;
      fp.Sp = (int)vt_len(pr);
      fp.q = Qc;
      fp.k = Kc;
      fp.v = Vt;
      fp.o = Oc;
      fp.o_lo = OLc;  // [S][hc][D]
      fp.H = pr.hc;
      fp.lse = Lrec;
      fp.S = S;
      fp.hc = pr.hc;
      fp.heads_per_kv = pr.heads_per_kv;
      fp.n_qtiles = n_fwd_tiles;
      fp.causal = pr.causal;
      fp.doc_off = nullptr;
      fp.n_docs = 0;
      fp.scale_log2 = scale * kLog2e;
      timed(K_FWD, st, [&] {
        launch_attn_fwd_bf16<D>(fp, st);
      });
      lo_v = RowsView<bf16>{OLc, (int64_t)pr.hc * D, D};
      lse_c = Lrec;
    } else {
      const size_t nq = (size_t)S * pr.hc * (D / 8);
      timed(K_PACK, st, [&] {
        hipLaunchKernelGGL(pack_heads_kernel, dim3(copy_grid(nq)), dim3(256), 0, st, (const uint4*)out, (uint4*)Oc,
                           S, pr.Hq, c.q_head0, pr.hc, D / 8);
      });
      lse_c = lse + (size_t)c.q_head0 * S;
    }
    constexpr int kRowsPerPreBlock = 256 / (D / 8);
    const unsigned pre_grid =
        (unsigned)std::min<size_t>(((size_t)S * pr.hc + kRowsPerPreBlock - 1) / kRowsPerPreBlock, 256 * 32);
    timed(K_BWD_PRE, st, [&] {
      hipLaunchKernelGGL((bwd_pre_kernel<bf16, D>), dim3(pre_grid), dim3(256), 0, st, RowsView<bf16>{Oc, D, SD},
                         lo_v, RowsView<bf16>{dOc, D, SD}, lse_c, (bf16*)nullptr, nDc, L2c, S, pr.hc);
    });
    BwdParams<bf16> bp;
    bp.q = Qc;
    bp.k = Kc;
    bp.v = Vc;
    bp.dout = dOc;
    bp.lse = lse_c;
    bp.negD = nDc;
    bp.lse2 = L2c;
    bp.dq = dQc;
    bp.dk_acc = dKa;
    bp.dv_acc = dVa;
    bp.dk_out = dKc;  // [S][nkv][D]
    bp.dv_out = dVc;
    bp.Hkv_total = c.n_kv;
    bp.S = S;
    bp.hc = pr.hc;
    bp.heads_per_kv = pr.heads_per_kv;
    bp.nkv = pr.nkv;
    bp.n_qtiles = n_qtiles;
    bp.n_ktiles = n_ktiles;
    bp.causal = pr.causal;
    bp.doc_off = nullptr;
    bp.n_docs = 0;
    bp.acc_load = !c.first_for_kv;
    bp.finalize = c.last_for_kv;
    bp.scale = scale;
    bp.scale_log2 = scale * kLog2e;
    timed(K_BWD_DKDV, st, [&] {
      hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D>), dim3(n_ktiles * pr.nkv), dim3(256), 0, st, bp);
    });
    timed(K_BWD_DQ, st, [&] {
      launch_attn_dq_bf16<D>(bp, st);
    });
    if (int rc = check_launch("attention block backward chunk")) return rc;

    // dWo's columns of the chunk's heads = dy^T o: [M = Dm][N = hc*D], K = tokens
    const GemmOperand o_tok = operand(Oc, D, 0, D, SD), o_tail = operand(Oc + (int64_t)K0 * D, D, 0, D, SD, tail);
    if (int rc = gemm_over_tokens(dy_tok, dy_tail, o_tok, o_tail, gemm_out(dwo + (int64_t)c.q_head0 * D,
                                  (int64_t)pr.Hq * D), Dm, pr.hc * D, S, split_buf, st))
      return rc;
    // dWq rows of the chunk's heads = dq^T x: [M = hc*D][N = Dm]
    const GemmOperand dq_tok = operand(dQc, D, 0, D, SD), dq_tail = operand(dQc + (int64_t)K0 * D, D, 0, D, SD, tail);
    if (int rc = gemm_over_tokens(dq_tok, dq_tail, x_tok, x_tail, gemm_out(dwq + (int64_t)c.q_head0 * D * Dm,
                                  (int64_t)Dm), pr.hc * D, Dm, S, split_buf, st))
      return rc;
    if (c.last_for_kv) {
      const int64_t ldk = (int64_t)c.n_kv * D;  // dk, dv rows: [S][nkv][D]
      const GemmOperand dk_tok = operand(dKc, ldk, 0), dk_tail = operand(dKc + K0 * ldk, ldk, 0, kUnblocked, 0, tail);
      const GemmOperand dv_tok = operand(dVc, ldk, 0), dv_tail = operand(dVc + K0 * ldk, ldk, 0, kUnblocked, 0, tail);
      if (int rc = gemm_over_tokens(dk_tok, dk_tail, x_tok, x_tail,
                                    gemm_out(dwk + (int64_t)c.kv_head0 * D * Dm, (int64_t)Dm), c.n_kv * D, Dm, S, split_buf, st))
        return rc;
      if (int rc = gemm_over_tokens(dv_tok, dv_tail, x_tok, x_tail,
                                    gemm_out(dwv + (int64_t)c.kv_head0 * D * Dm, (int64_t)Dm), c.n_kv * D, Dm, S, split_buf, st))
        return rc;
    }
    // dx (+)= dq_h Wq_h for the chunk's heads of each kv group, then, once
    // the group's dk and dv are final, dk_g Wk_g + dv_g Wv_g: one fixed order
    // for every head_chunk, so dx's fp32 sums do not depend on it
    GemmOut<float> dxo = gemm_out(dx, Dm);
    const int groups = pr.hc >= pr.G ? c.n_kv : 1;
    for (int gl = 0; gl < groups; ++gl) {
      for (int j = 0; j < pr.heads_per_kv; ++j) {
        const int hl = gl * pr.heads_per_kv + j, h = c.q_head0 + hl;
        const GemmOperand wqh = operand(reinterpret_cast<const bf16*>(wq) + (int64_t)h * D * Dm, Dm, 0);
        timed(K_GEMM, st, [&] { (void)gemm(operand(dQc + hl * SD, D, 1), wqh, dxo, S, Dm, D, dx_started, st); });
        dx_started = true;
      }
      if (c.last_for_kv) {
        const int64_t ldk = (int64_t)c.n_kv * D;
        const int g = c.kv_head0 + gl;
        const GemmOperand wkg = operand(reinterpret_cast<const bf16*>(wk) + (int64_t)g * D * Dm, Dm, 0);
        const GemmOperand wvg = operand(reinterpret_cast<const bf16*>(wv) + (int64_t)g * D * Dm, Dm, 0);
        timed(K_GEMM, st, [&] { (void)gemm(operand(dKc + gl * D, ldk, 1), wkg, dxo, S, Dm, D, 1, st); });
        timed(K_GEMM, st, [&] { (void)gemm(operand(dVc + gl * D, ldk, 1), wvg, dxo, S, Dm, D, 1, st); });
      }
    }
    if (int rc = check_launch("attention block backward projections")) return rc;
  }
  return UPIPE_OK;
}

// ---------------------------------------------------------------------------
// Sequence-tiled cross-entropy (loss_kernels.hpp). Pool: one tile's fp32
// logits [tile][Vp] and its bf16 gradient rows [tile][Vp], Vp = V rounded up
// to 64 (zero columns past V), reused by every tile.
// ---------------------------------------------------------------------------
int64_t vocab_pad(int V) { return ((int64_t)V + 63) / 64 * 64; }
struct LossPool {
  size_t logits, g, total;
};
LossPool loss_pool(int tile, int V, bool grad) {
  LossPool p;
  size_t off = 0;
  p.logits = off; off += align_up((size_t)tile * vocab_pad(V) * 4);
  p.g = off; off += grad ? align_up((size_t)tile * vocab_pad(V) * 2) : 0;
  p.total = off;
  return p;
}

int validate_loss(int64_t S, int Dm, int V, int tile) {
  if (S < 1 || S >= (1ll << 31)) return fail(UPIPE_EINVAL, "S must be in [1, 2^31) (got %lld)", (long long)S);
  if (Dm < 64 || Dm % 64) return fail(UPIPE_EUNSUPPORTED, "model dim Dm (%d) must be a positive multiple of 64", Dm);
  if (V < 8 || V % 8) return fail(UPIPE_EUNSUPPORTED, "vocabulary size V (%d) must be a positive multiple of 8", V);
  if (tile < 64 || tile % 64) return fail(UPIPE_EINVAL, "tile (%d) must be a positive multiple of 64", tile);
  if ((uint64_t)tile * vocab_pad(V) * 4 >= (1ull << 40)) return fail(UPIPE_EUNSUPPORTED, "tile x V too large");
  return UPIPE_OK;
}

int run_ce_loss(const bf16* h, const bf16* w, const int32_t* labels, float* loss, bf16* dh, float* dw, int64_t S64,
                int Dm, int V, int tile, float scale, char* ws, hipStream_t st) {
  const bool grad = dh || dw;
  const LossPool pool = loss_pool(tile, V, grad);
  const int S = (int)S64;
  const int64_t Vp = vocab_pad(V);
  float* logits = reinterpret_cast<float*>(ws + pool.logits);
  bf16* G = grad ? reinterpret_cast<bf16*>(ws + pool.g) : nullptr;
  const GemmOperand wk = operand(w, Dm, 1);  // W [V][Dm]: logits = h W^T
  // W as [K = V][N = Dm] for dh = G W, K padded to Vp: rows past V are read as
  // row V - 1, against G's zero columns
  const GemmOperand wn = operand(w, Dm, 0, kUnblocked, 0, V);
  const GemmOperand gk = operand(G, Vp, 1);  // G [tile][Vp], K = vocab contiguous
  const GemmOperand gm = operand(G, Vp, 0);  // G^T: M = vocab contiguous, K = token (zero rows past T)
  for (int t0 = 0; t0 < S; t0 += tile) {
    const int T = std::min(tile, S - t0);
    const GemmOperand hk = operand(h + (int64_t)t0 * Dm, Dm, 1);  // the tile's rows of h, K = Dm
    // as [K = token][N = Dm] for dW = G^T h, K padded to the tile: tokens past
    // T are read as token T - 1, against G's zero rows
    const GemmOperand hn = operand(h + (int64_t)t0 * Dm, Dm, 0, kUnblocked, 0, T);
    GemmOut<float> lo = gemm_out(logits, Vp);
    timed(K_GEMM, st, [&] { (void)gemm(hk, wk, lo, T, V, Dm, 0, st); });
    timed(K_CE_ROWS, st, [&] {
      hipLaunchKernelGGL(ce_rows_kernel, dim3(grad ? tile : T), dim3(256), 0, st, logits, (int)Vp, labels + t0,
                         loss + t0, G, (int)Vp, T, V, scale);
    });
    if (dh) {
      GemmOut<bf16> o = gemm_out(dh + (int64_t)t0 * Dm, (int64_t)Dm);
      timed(K_GEMM, st, [&] { (void)gemm(gk, wn, o, T, Dm, (int)Vp, 0, st); });
    }
    if (dw) {
      GemmOut<float> o = gemm_out(dw, (int64_t)Dm);
      timed(K_GEMM, st, [&] { (void)gemm(gm, hn, o, V, Dm, tile, t0 > 0, st); });
    }
    if (int rc = check_launch("cross-entropy tile")) return rc;
  }
  return UPIPE_OK;
}

// ---------------------------------------------------------------------------
// Sequence-tiled SwiGLU MLP (mlp_kernels.hpp). Pool: one tile's gate and up
// rows g, u and activation a [tile][F] bf16, and for the backward the fp32
// da [tile][F]; reused by every tile, independent of S.
// ---------------------------------------------------------------------------
struct MlpPool {
  size_t g, u, a, da, total;
};
MlpPool mlp_pool(int F, int tile, bool grad) {
  const size_t B = (size_t)tile * F * 2;
  MlpPool p;
  size_t off = 0;
  p.g = off; off += align_up(B);
  p.u = off; off += align_up(B);
  p.a = off; off += align_up(B);
  p.da = off; off += grad ? align_up(2 * B) : 0;
  p.total = off;
  return p;
}

int validate_mlp(int64_t S, int Dm, int F, int tile) {
  if (S < 1 || S >= (1ll << 31)) return fail(UPIPE_EINVAL, "S must be in [1, 2^31) (got %lld)", (long long)S);
  if (Dm < 64 || Dm % 64) return fail(UPIPE_EUNSUPPORTED, "model dim Dm (%d) must be a positive multiple of 64", Dm);
  if (F < 64 || F % 64) return fail(UPIPE_EUNSUPPORTED, "hidden dim F (%d) must be a positive multiple of 64", F);
  if (tile < 64 || tile % 64) return fail(UPIPE_EINVAL, "tile (%d) must be a positive multiple of 64", tile);
  if ((uint64_t)tile * F * 10 >= (1ull << 40)) return fail(UPIPE_EUNSUPPORTED, "tile x F too large");
  return UPIPE_OK;
}

// g, u and a of one tile of T tokens starting at token t0 (rows T..tile-1 of a
// zeroed when zero_tail); returns the launch status.
int mlp_tile_forward(const bf16* x, const bf16* wg, const bf16* wu, int t0, int T, int Dm, int F, int tile,
                     const MlpPool& pool, char* ws, bool zero_tail, hipStream_t st) {
  bf16* g = reinterpret_cast<bf16*>(ws + pool.g);
  bf16* u = reinterpret_cast<bf16*>(ws + pool.u);
  bf16* a = reinterpret_cast<bf16*>(ws + pool.a);
  const GemmOperand xk = operand(x + (int64_t)t0 * Dm, Dm, 1);  // the tile's rows of x, K = Dm
  timed(K_GEMM, st, [&] { (void)gemm(xk, operand(wg, Dm, 1), gemm_out(g, (int64_t)F), T, F, Dm, 0, st); });
  timed(K_GEMM, st, [&] { (void)gemm(xk, operand(wu, Dm, 1), gemm_out(u, (int64_t)F), T, F, Dm, 0, st); });
  timed(K_SWIGLU, st, [&] {
    hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(zero_tail ? tile : T), dim3(256), 0, st, g, u, a, T, F);
  });
  return check_launch("swiglu forward");
}

int run_mlp_fwd(const bf16* x, const bf16* wg, const bf16* wu, const bf16* wd, bf16* y, int S, int Dm, int F,
                int tile, char* ws, hipStream_t st) {
  const MlpPool pool = mlp_pool(F, tile, false);
  const bf16* a = reinterpret_cast<const bf16*>(ws + pool.a);
  for (int t0 = 0; t0 < S; t0 += tile) {
    const int T = std::min(tile, S - t0);
    if (int rc = mlp_tile_forward(x, wg, wu, t0, T, Dm, F, tile, pool, ws, false, st)) return rc;
    // y = a Wd^T: Wd [Dm][F] is k-major
    timed(K_GEMM, st, [&] {
      (void)gemm(operand(a, F, 1), operand(wd, F, 1), gemm_out(y + (int64_t)t0 * Dm, (int64_t)Dm), T, Dm, F, 0, st);
    });
    if (int rc = check_launch("MLP tile")) return rc;
  }
  return UPIPE_OK;
}

int run_mlp_bwd(const bf16* x, const bf16* wg, const bf16* wu, const bf16* wd, const bf16* dy, float* dx, float* dwg,
                float* dwu, float* dwd, int S, int Dm, int F, int tile, char* ws, hipStream_t st) {
  const MlpPool pool = mlp_pool(F, tile, true);
  bf16* g = reinterpret_cast<bf16*>(ws + pool.g);  // becomes dg
  bf16* u = reinterpret_cast<bf16*>(ws + pool.u);  // becomes du
  const bf16* a = reinterpret_cast<const bf16*>(ws + pool.a);
  float* da = reinterpret_cast<float*>(ws + pool.da);
  for (int t0 = 0; t0 < S; t0 += tile) {
    const int T = std::min(tile, S - t0);
    // the tile's forward again (activations are not kept across the sequence)
    if (int rc = mlp_tile_forward(x, wg, wu, t0, T, Dm, F, tile, pool, ws, true, st)) return rc;
    const bf16* dyt = dy + (int64_t)t0 * Dm;
    const bf16* xt = x + (int64_t)t0 * Dm;
    // da = dy Wd: Wd read as [K = Dm][N = F], N contiguous
    timed(K_GEMM, st, [&] {
      (void)gemm(operand(dyt, Dm, 1), operand(wd, F, 0), gemm_out(da, (int64_t)F), T, F, Dm, 0, st);
    });
    timed(K_SWIGLU, st, [&] { hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(tile), dim3(256), 0, st, da, g, u, T, F); });
    // dx = dg Wg + du Wu: Wg, Wu read as [K = F][N = Dm]
    float* dxt = dx + (int64_t)t0 * Dm;
    timed(K_GEMM, st, [&] {
      (void)gemm(operand(g, F, 1), operand(wg, Dm, 0), gemm_out(dxt, (int64_t)Dm), T, Dm, F, 0, st);
    });
    timed(K_GEMM, st, [&] {
      (void)gemm(operand(u, F, 1), operand(wu, Dm, 0), gemm_out(dxt, (int64_t)Dm), T, Dm, F, 1, st);
    });
    // weight gradients, summed over tiles in order: K = the tile's tokens,
    // padded to the tile; the token-major x and dy rows past T are read as row
    // T - 1 against the zero rows of dg, du and a
    const GemmOperand xn = operand(xt, Dm, 0, kUnblocked, 0, T);     // [K = token][N = Dm]
    const GemmOperand dym = operand(dyt, Dm, 0, kUnblocked, 0, T);   // [K = token][M = Dm]
    timed(K_GEMM, st, [&] {
      (void)gemm(operand(g, F, 0), xn, gemm_out(dwg, (int64_t)Dm), F, Dm, tile, t0 > 0, st);
    });
    timed(K_GEMM, st, [&] {
      (void)gemm(operand(u, F, 0), xn, gemm_out(dwu, (int64_t)Dm), F, Dm, tile, t0 > 0, st);
    });
    timed(K_GEMM, st, [&] {
      (void)gemm(dym, operand(a, F, 0), gemm_out(dwd, (int64_t)F), Dm, F, tile, t0 > 0, st);
    });
    if (int rc = check_launch("MLP backward tile")) return rc;
  }
  return UPIPE_OK;
}

}  // namespace
}  // namespace upipe

using namespace upipe;

extern "C" {

size_t upipe_attn_fwd_workspace_bytes(int64_t S, int Hq, int Hkv, int d, int head_chunk, int dtype) {
  Problem pr;
  if (validate(S, Hq, Hkv, d, head_chunk, 1, dtype, &pr) != UPIPE_OK) return 0;
  g_error.clear();
  return fwd_pool(pr).total;
}

size_t upipe_attn_bwd_workspace_bytes(int64_t S, int Hq, int Hkv, int d, int head_chunk, int dtype) {
  Problem pr;
  if (validate(S, Hq, Hkv, d, head_chunk, 1, dtype, &pr) != UPIPE_OK) return 0;
  g_error.clear();
  return bwd_pool(pr).total;
}

size_t upipe_attn_workspace_bytes(int64_t S, int Hq, int Hkv, int d, int head_chunk, int dtype) {
  Problem pr;
  if (validate(S, Hq, Hkv, d, head_chunk, 1, dtype, &pr) != UPIPE_OK) return 0;
  g_error.clear();
  return std::max(fwd_pool(pr).total, bwd_pool(pr).total);
}

size_t upipe_attn_bwd_fused_workspace_bytes(int64_t S, int Hq, int Hkv, int d, int head_chunk) {
  Problem pr;
  if (validate(S, Hq, Hkv, d, head_chunk, 1, UPIPE_BF16, &pr) != UPIPE_OK) return 0;
  if (validate_fused(pr) != UPIPE_OK) return 0;
  g_error.clear();
  return fused_pool(pr).total;
}

int upipe_attn_pick_head_chunk(int64_t S, int Hq, int Hkv, int d, int dtype, size_t budget_bytes) {
  Problem pr;
  if (int rc = validate(S, Hq, Hkv, d, 1, 1, dtype, &pr)) return rc;
  // Every valid chunk size is tried: the pools are not monotone in hc (a
  // chunk of a whole kv group drops the fp32 dK/dV accumulators, so at G = 2
  // in bf16 head_chunk 2 needs less than 1).
  int best = 0, min_hc = 0;
  size_t min_need = 0;
  for (int hc = 1; hc <= Hq; ++hc) {
    if (validate(S, Hq, Hkv, d, hc, 1, dtype, &pr) != UPIPE_OK) continue;  // not a valid chunk size
    const size_t need = std::max(fwd_pool(pr).total, bwd_pool(pr).total);
    if (!min_hc || need < min_need) {
      min_hc = hc;
      min_need = need;
    }
    if (need <= budget_bytes) best = hc;
  }
  if (!best)
    return fail(UPIPE_EWORKSPACE, "no head_chunk fits: the smallest workspace is %zu bytes (head_chunk %d), budget %zu",
                min_need, min_hc, budget_bytes);
  g_error.clear();
  return best;
}

}  // extern "C"

// Scratch for upipe_attn_fwd_noalloc: the forward's fixed buffer pool in a
// file-scope device array, so that entry point never allocates. Each GPU the
// library runs on holds its own copy from the first call until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// its device address is looked up once per device (with that device current)
// and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[UPIPE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = UPIPE_NOALLOC_SCRATCH_BYTES;
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_addr;  // per device ordinal; null until looked up

int scratch_address(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(UPIPE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_addr.size() <= dev) g_scratch_addr.resize(dev + 1, nullptr);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(UPIPE_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return UPIPE_OK;
}

// Packed-document arguments: a device array of n_docs + 1 offsets, or none.
int validate_docs(const int32_t* doc_offsets, int n_docs, Problem* pr) {
  if (!doc_offsets) return fail(UPIPE_EINVAL, "doc_offsets is NULL");
  if (n_docs < 1) return fail(UPIPE_EINVAL, "n_docs must be >= 1 (got %d)", n_docs);
  if (reinterpret_cast<uintptr_t>(doc_offsets) % 4) return fail(UPIPE_EINVAL, "doc_offsets is not 4-byte aligned");
  pr->doc_off = doc_offsets;
  pr->n_docs = n_docs;
  return UPIPE_OK;
}

int fwd_entry(const void* q, const void* k, const void* v, void* out, void* out_lo, float* lse, int64_t S, int Hq,
              int Hkv, int d, int head_chunk, int causal, const int32_t* doc_offsets, int n_docs, int dtype,
              void* workspace, size_t workspace_bytes, void* stream) {
  Problem pr;
  if (int rc = validate(S, Hq, Hkv, d, head_chunk, causal, dtype, &pr)) return rc;
  if (doc_offsets || n_docs)
    if (int rc = validate_docs(doc_offsets, n_docs, &pr)) return rc;
  const void* ptrs[] = {q, k, v, out, lse, workspace};
  const char* names[] = {"q", "k", "v", "out", "lse", "workspace"};
  for (int i = 0; i < 6; ++i) {
    if (!ptrs[i]) return fail(UPIPE_EINVAL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  if (out_lo && !aligned16(out_lo)) return fail(UPIPE_EINVAL, "out_lo is not 16-byte aligned");
  if (dtype != UPIPE_BF16) out_lo = nullptr;  // fp32 outputs carry no rounding residual
  const size_t need = fwd_pool(pr).total;
  if (workspace_bytes < need)
    return fail(UPIPE_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  g_error.clear();
  (void)hipGetLastError();  // launch errors are checked after each chunk; drop any older one first
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16) {
    if (d == 128) return run_fwd<bf16, 128>(pr, q, k, v, out, out_lo, lse, ws, st);
    return run_fwd<bf16, 64>(pr, q, k, v, out, out_lo, lse, ws, st);
  }
  if (d == 128) return run_fwd<float, 128>(pr, q, k, v, out, out_lo, lse, ws, st);
  return run_fwd<float, 64>(pr, q, k, v, out, out_lo, lse, ws, st);
}

int bwd_entry(const void* q, const void* k, const void* v, const void* out, const void* out_lo, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, int64_t S, int Hq, int Hkv, int d, int head_chunk,
              int causal, const int32_t* doc_offsets, int n_docs, int dtype, void* workspace,
              size_t workspace_bytes, void* stream) {
  Problem pr;
  if (int rc = validate(S, Hq, Hkv, d, head_chunk, causal, dtype, &pr)) return rc;
  if (doc_offsets || n_docs)
    if (int rc = validate_docs(doc_offsets, n_docs, &pr)) return rc;
  const void* ptrs[] = {q, k, v, out, dout, lse, dq, dk, dv, workspace};
  const char* names[] = {"q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "workspace"};
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) return fail(UPIPE_EINVAL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  if (out_lo && !aligned16(out_lo)) return fail(UPIPE_EINVAL, "out_lo is not 16-byte aligned");
  if (dtype != UPIPE_BF16) out_lo = nullptr;
  const size_t need = bwd_pool(pr).total;
  if (workspace_bytes < need)
    return fail(UPIPE_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  g_error.clear();
  (void)hipGetLastError();  // launch errors are checked after each chunk; drop any older one first
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16) {
    if (d == 128) return run_bwd<bf16, 128>(pr, q, k, v, out, out_lo, dout, lse, dq, dk, dv, ws, st);
    return run_bwd<bf16, 64>(pr, q, k, v, out, out_lo, dout, lse, dq, dk, dv, ws, st);
  }
  if (d == 128) return run_bwd<float, 128>(pr, q, k, v, out, out_lo, dout, lse, dq, dk, dv, ws, st);
  return run_bwd<float, 64>(pr, q, k, v, out, out_lo, dout, lse, dq, dk, dv, ws, st);
}

}  // namespace

extern "C" {

int upipe_attn_fwd(const void* q, const void* k, const void* v, void* out, void* out_lo, float* lse, int64_t S,
                   int Hq, int Hkv, int d, int head_chunk, int causal, int dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return fwd_entry(q, k, v, out, out_lo, lse, S, Hq, Hkv, d, head_chunk, causal, nullptr, 0, dtype, workspace,
                   workspace_bytes, stream);
}

int upipe_attn_fwd_docs(const void* q, const void* k, const void* v, void* out, void* out_lo, float* lse,
                        int64_t S, int Hq, int Hkv, int d, int head_chunk, int causal, const int32_t* doc_offsets,
                        int n_docs, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!doc_offsets && !n_docs) return fail(UPIPE_EINVAL, "doc_offsets is NULL");
  return fwd_entry(q, k, v, out, out_lo, lse, S, Hq, Hkv, d, head_chunk, causal, doc_offsets, n_docs, dtype,
                   workspace, workspace_bytes, stream);
}

int upipe_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* out_lo,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv, int64_t S, int Hq, int Hkv,
                   int d, int head_chunk, int causal, int dtype, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return bwd_entry(q, k, v, out, out_lo, dout, lse, dq, dk, dv, S, Hq, Hkv, d, head_chunk, causal, nullptr, 0,
                   dtype, workspace, workspace_bytes, stream);
}

int upipe_attn_bwd_fused(const void* q, const void* k, const void* v, const void* out, const void* out_lo,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int64_t S, int Hq,
                         int Hkv, int d, int head_chunk, int causal, int max_polls, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Problem pr;
  if (int rc = validate(S, Hq, Hkv, d, head_chunk, causal, UPIPE_BF16, &pr)) return rc;
  if (int rc = validate_fused(pr)) return rc;
  const void* ptrs[] = {q, k, v, out, dout, lse, dq, dk, dv, workspace};
  const char* names[] = {"q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv", "workspace"};
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) return fail(UPIPE_EINVAL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  if (out_lo && !aligned16(out_lo)) return fail(UPIPE_EINVAL, "out_lo is not 16-byte aligned");
  if (max_polls < 0) return fail(UPIPE_EINVAL, "max_polls must be >= 0 (got %d)", max_polls);
  const size_t need = fused_pool(pr).total;
  if (workspace_bytes < need)
    return fail(UPIPE_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  g_error.clear();
  (void)hipGetLastError();
  return run_bwd_fused<128>(pr, q, k, v, out, out_lo, dout, lse, dq, dk, dv, reinterpret_cast<char*>(workspace),
                            max_polls ? max_polls : kDefaultMaxPolls, reinterpret_cast<hipStream_t>(stream));
}

int upipe_attn_bwd_docs(const void* q, const void* k, const void* v, const void* out, const void* out_lo,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int64_t S, int Hq,
                        int Hkv, int d, int head_chunk, int causal, const int32_t* doc_offsets, int n_docs,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!doc_offsets && !n_docs) return fail(UPIPE_EINVAL, "doc_offsets is NULL");
  return bwd_entry(q, k, v, out, out_lo, dout, lse, dq, dk, dv, S, Hq, Hkv, d, head_chunk, causal, doc_offsets,
                   n_docs, dtype, workspace, workspace_bytes, stream);
}

int upipe_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, void* out_lo, float* lse,
                           int64_t S, int Hq, int Hkv, int d, int head_chunk, int causal, int dtype,
                           void* stream) {
  Problem pr;
  if (int rc = validate(S, Hq, Hkv, d, head_chunk, causal, dtype, &pr)) return rc;
  const size_t need = fwd_pool(pr).total;
  if (need > kScratchBytes)
    return fail(UPIPE_EWORKSPACE, "forward pool needs %zu bytes, more than the %zu-byte static scratch array", need,
                kScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_address(&ws)) return rc;
  return fwd_entry(q, k, v, out, out_lo, lse, S, Hq, Hkv, d, head_chunk, causal, nullptr, 0, dtype, ws, kScratchBytes,
                   stream);
}

int upipe_gemm_bf16(const void* a, int64_t lda, int64_t a_blk, int64_t a_blk_stride, int a_kmajor, const void* b,
                    int64_t ldb, int64_t b_blk, int64_t b_blk_stride, int b_kmajor, void* c, int64_t ldc,
                    int64_t c_blk, int64_t c_blk_stride, int c_dtype, int accumulate, int M, int N, int K,
                    void* stream) {
  if (M < 1 || N < 1 || K < 1) return fail(UPIPE_EINVAL, "M, N, K must be >= 1 (got %d, %d, %d)", M, N, K);
  if (K % 64) return fail(UPIPE_EUNSUPPORTED, "K (%d) must be a multiple of 64", K);
  if (N % 8) return fail(UPIPE_EUNSUPPORTED, "N (%d) must be a multiple of 8", N);
  if (c_dtype != UPIPE_BF16 && c_dtype != UPIPE_FP32) return fail(UPIPE_EUNSUPPORTED, "unsupported C dtype %d", c_dtype);
  if (accumulate && c_dtype != UPIPE_FP32) return fail(UPIPE_EINVAL, "accumulate needs an fp32 C");
  const GemmOperand ao = operand(a, lda, a_kmajor != 0, a_blk > 0 ? a_blk : kUnblocked, a_blk_stride);
  const GemmOperand bo = operand(b, ldb, b_kmajor != 0, b_blk > 0 ? b_blk : kUnblocked, b_blk_stride);
  if (int rc = check_operand("a", ao, M, K)) return rc;
  if (int rc = check_operand("b", bo, N, K)) return rc;
  if (!c) return fail(UPIPE_EINVAL, "c is NULL");
  if ((uintptr_t)c % 16) return fail(UPIPE_EINVAL, "c is not 16-byte aligned");
  const int64_t cb = c_blk > 0 ? c_blk : kUnblocked;
  if (ldc < 1 || ldc % 8 || block_shift(cb) < 3 || (cb < kUnblocked && c_blk_stride % 8))
    return fail(UPIPE_EINVAL, "c: ldc and block stride must be multiples of 8, the block length a power of two >= 8");
  g_error.clear();
  (void)hipGetLastError();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int rc;
  timed(K_GEMM, st, [&] {
    if (c_dtype == UPIPE_FP32)
      rc = gemm(ao, bo, gemm_out(reinterpret_cast<float*>(c), ldc, cb, c_blk_stride), M, N, K, accumulate, st);
    else
      rc = gemm(ao, bo, gemm_out(reinterpret_cast<bf16*>(c), ldc, cb, c_blk_stride), M, N, K, 0, st);
  });
  return rc;
}

size_t upipe_attn_block_fwd_workspace_bytes(int64_t S, int Dm, int Hq, int Hkv, int d, int head_chunk) {
  Problem pr;
  if (validate_block(S, Dm, Hq, Hkv, d, head_chunk, 1, &pr) != UPIPE_OK) return 0;
  g_error.clear();
  return block_pool(pr).total;
}

int upipe_attn_block_fwd(const void* x, const void* wq, const void* wk, const void* wv, const void* wo, float* y,
                         void* out, float* lse, int64_t S, int Dm, int Hq, int Hkv, int d, int head_chunk,
                         int causal, void* workspace, size_t workspace_bytes, void* stream) {
  Problem pr;
  if (int rc = validate_block(S, Dm, Hq, Hkv, d, head_chunk, causal, &pr)) return rc;
  const void* ptrs[] = {x, wq, wk, wv, wo, y, lse, workspace};
  const char* names[] = {"x", "wq", "wk", "wv", "wo", "y", "lse", "workspace"};
  for (int i = 0; i < 8; ++i) {
    if (!ptrs[i]) return fail(UPIPE_EINVAL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  if (out && !aligned16(out)) return fail(UPIPE_EINVAL, "out is not 16-byte aligned");
  const size_t need = block_pool(pr).total;
  if (workspace_bytes < need)
    return fail(UPIPE_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  g_error.clear();
  (void)hipGetLastError();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (d == 128) return run_block_fwd<128>(pr, Dm, x, wq, wk, wv, wo, y, out, lse, ws, st);
  return run_block_fwd<64>(pr, Dm, x, wq, wk, wv, wo, y, out, lse, ws, st);
}

size_t upipe_attn_block_bwd_workspace_bytes(int64_t S, int Dm, int Hq, int Hkv, int d, int head_chunk,
                                            int recompute) {
  Problem pr;
  if (validate_block(S, Dm, Hq, Hkv, d, head_chunk, 1, &pr) != UPIPE_OK) return 0;
  g_error.clear();
  return block_bwd_pool(pr, Dm, recompute != 0).total;
}

int upipe_attn_block_bwd(const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                         const void* dy, const void* out, const float* lse, float* dx, float* dwq, float* dwk,
                         float* dwv, float* dwo, int64_t S, int Dm, int Hq, int Hkv, int d, int head_chunk,
                         int causal, void* workspace, size_t workspace_bytes, void* stream) {
  Problem pr;
  if (int rc = validate_block(S, Dm, Hq, Hkv, d, head_chunk, causal, &pr)) return rc;
  const void* ptrs[] = {x, wq, wk, wv, wo, dy, dx, dwq, dwk, dwv, dwo, workspace};
  const char* names[] = {"x", "wq", "wk", "wv", "wo", "dy", "dx", "dwq", "dwk", "dwv", "dwo", "workspace"};
  for (int i = 0; i < 12; ++i) {
    if (!ptrs[i]) return fail(UPIPE_EINVAL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  if (out && !aligned16(out)) return fail(UPIPE_EINVAL, "out is not 16-byte aligned");
  if (out && !lse) return fail(UPIPE_EINVAL, "lse is NULL (it is required when out is given)");
  const size_t need = block_bwd_pool(pr, Dm, out == nullptr).total;
  if (workspace_bytes < need)
    return fail(UPIPE_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  g_error.clear();
  (void)hipGetLastError();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (d == 128)
    return run_block_bwd<128>(pr, Dm, x, wq, wk, wv, wo, dy, out, lse, dx, dwq, dwk, dwv, dwo, ws, st);
  return run_block_bwd<64>(pr, Dm, x, wq, wk, wv, wo, dy, out, lse, dx, dwq, dwk, dwv, dwo, ws, st);
}

size_t upipe_ce_loss_workspace_bytes(int64_t S, int Dm, int V, int tile, int with_grad) {
  if (validate_loss(S, Dm, V, tile) != UPIPE_OK) return 0;
  g_error.clear();
  return loss_pool(tile, V, with_grad != 0).total;
}

int upipe_ce_loss_tiled(const void* h, const void* w, const int32_t* labels, float* loss, void* dh, float* dw,
                        int64_t S, int Dm, int V, int tile, float grad_scale, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (int rc = validate_loss(S, Dm, V, tile)) return rc;
  const void* ptrs[] = {h, w, labels, loss, workspace};
  const char* names[] = {"h", "w", "labels", "loss", "workspace"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(UPIPE_EINVAL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  if ((dh && !aligned16(dh)) || (dw && !aligned16(dw))) return fail(UPIPE_EINVAL, "dh or dw is not 16-byte aligned");
  const size_t need = loss_pool(tile, V, dh || dw).total;
  if (workspace_bytes < need)
    return fail(UPIPE_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  g_error.clear();
  (void)hipGetLastError();
  return run_ce_loss(reinterpret_cast<const bf16*>(h), reinterpret_cast<const bf16*>(w), labels, loss,
                     reinterpret_cast<bf16*>(dh), dw, S, Dm, V, tile, grad_scale, reinterpret_cast<char*>(workspace),
                     reinterpret_cast<hipStream_t>(stream));
}

size_t upipe_mlp_workspace_bytes(int64_t S, int Dm, int F, int tile, int with_grad) {
  if (validate_mlp(S, Dm, F, tile) != UPIPE_OK) return 0;
  g_error.clear();
  return mlp_pool(F, tile, with_grad != 0).total;
}

int upipe_mlp_tiled_fwd(const void* x, const void* wg, const void* wu, const void* wd, void* y, int64_t S, int Dm,
                        int F, int tile, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = validate_mlp(S, Dm, F, tile)) return rc;
  const void* ptrs[] = {x, wg, wu, wd, y, workspace};
  const char* names[] = {"x", "wg", "wu", "wd", "y", "workspace"};
  for (int i = 0; i < 6; ++i) {
    if (!ptrs[i]) return fail(UPIPE_EINVAL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  const size_t need = mlp_pool(F, tile, false).total;
  if (workspace_bytes < need)
    return fail(UPIPE_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  g_error.clear();
  (void)hipGetLastError();
  return run_mlp_fwd(reinterpret_cast<const bf16*>(x), reinterpret_cast<const bf16*>(wg),
                     reinterpret_cast<const bf16*>(wu), reinterpret_cast<const bf16*>(wd), reinterpret_cast<bf16*>(y),
                     (int)S, Dm, F, tile, reinterpret_cast<char*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

int upipe_mlp_tiled_bwd(const void* x, const void* wg, const void* wu, const void* wd, const void* dy, float* dx,
                        float* dwg, float* dwu, float* dwd, int64_t S, int Dm, int F, int tile, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (int rc = validate_mlp(S, Dm, F, tile)) return rc;
  const void* ptrs[] = {x, wg, wu, wd, dy, dx, dwg, dwu, dwd, workspace};
  const char* names[] = {"x", "wg", "wu", "wd", "dy", "dx", "dwg", "dwu", "dwd", "workspace"};
  for (int i = 0; i < 10; ++i) {
    if (!ptrs[i]) return fail(UPIPE_EINVAL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(UPIPE_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  const size_t need = mlp_pool(F, tile, true).total;
  if (workspace_bytes < need)
    return fail(UPIPE_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  g_error.clear();
  (void)hipGetLastError();
  return run_mlp_bwd(reinterpret_cast<const bf16*>(x), reinterpret_cast<const bf16*>(wg),
                     reinterpret_cast<const bf16*>(wu), reinterpret_cast<const bf16*>(wd),
                     reinterpret_cast<const bf16*>(dy), dx, dwg, dwu, dwd, (int)S, Dm, F, tile,
                     reinterpret_cast<char*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

int upipe_attn_plan(int Hq, int Hkv, int head_chunk, int max_chunks, int32_t* q_head0, int32_t* kv_head0,
                    int32_t* n_kv, int32_t* flags) {
  Problem pr;
  if (int rc = validate(1, Hq, Hkv, 64, head_chunk, 1, UPIPE_BF16, &pr)) return rc;
  const std::vector<Chunk> cs = plan(pr);
  if (max_chunks < (int)cs.size())
    return fail(UPIPE_EINVAL, "max_chunks (%d) smaller than the chunk count (%d)", max_chunks, (int)cs.size());
  for (size_t i = 0; i < cs.size(); ++i) {
    if (q_head0) q_head0[i] = cs[i].q_head0;
    if (kv_head0) kv_head0[i] = cs[i].kv_head0;
    if (n_kv) n_kv[i] = cs[i].n_kv;
    if (flags) flags[i] = (cs[i].load_kv ? 1 : 0) | (cs[i].first_for_kv ? 2 : 0) | (cs[i].last_for_kv ? 4 : 0);
  }
  g_error.clear();
  return (int)cs.size();
}

int upipe_profile_enable(int on) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof.on = on != 0;
  return UPIPE_OK;
}

int upipe_profile_read(int max_kernels, const char** names, int64_t* launches, double* total_ms) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  if (int rc = profile_flush()) return rc;
  int n = 0;
  for (int i = 0; i < K_COUNT; ++i) {
    if (!g_prof.launches[i]) continue;
    if (n < max_kernels) {
      if (names) names[n] = kKernelNames[i];
      if (launches) launches[n] = g_prof.launches[i];
      if (total_ms) total_ms[n] = g_prof.ms[i];
    }
    ++n;
  }
  return n;
}

int upipe_profile_completed(int* total) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  int done = 0;
  for (const Profiler::Rec& r : g_prof.pending) {
    if (hipEventQuery(r.b) != hipSuccess) break;  // launches complete in stream order
    ++done;
  }
  if (total) *total = (int)g_prof.pending.size();
  return done;
}

void upipe_profile_reset(void) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  for (Profiler::Rec& r : g_prof.pending) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.pending.clear();
  for (int i = 0; i < K_COUNT; ++i) {
    g_prof.launches[i] = 0;
    g_prof.ms[i] = 0;
  }
}

const char* upipe_last_error(void) { return g_error.c_str(); }

}  // extern "C"
