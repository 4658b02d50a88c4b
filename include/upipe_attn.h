/*
 * upipe_attn.h -- C ABI of the MI355X (gfx950) UPipe causal GQA attention library.
 *
 * What the library computes. Exact softmax attention, forward and backward,
 * for one GPU's share of heads over the whole sequence, as under Ulysses-style
 * context parallelism, where each GPU owns whole heads and runs attention over
 * every position for them ("Road to 5 Million Tokens" talk summary, Chapters:
 * the DeepSpeed Ulysses chapter; the talk digest's Quiz answer on Ulysses).
 * Masking is causal: a query position attends to itself and to every earlier
 * position (MaxText long-context article, the section on where long-sequence
 * training gets stuck). Query heads may share key/value heads (GQA, named in
 * the same article's release section): query head h reads kv head
 * h / (Hq/Hkv) (contiguous groups).
 *
 *   s_ij  = tau * <q_hi, k_gj>,  tau = 1/sqrt(d)
 *   lse_hi = ln sum_{j<=i} exp(s_ij)          (j over all keys if causal == 0)
 *   out_hi = sum_{j<=i} exp(s_ij - lse_hi) v_gj
 *
 * How it runs (UPipe). The heads are processed in sequential chunks of
 * head_chunk heads; every chunk reuses the same buffers of one fixed pool
 * (the workspace) instead of allocating buffers for all heads at once (talk
 * summary, Chapters: the chapter on processing heads in batches; talk digest,
 * Quiz answer on U-Pipe). Peak device memory therefore grows with head_chunk,
 * not with Hq. Per chunk: the chunk's heads are copied from the caller's
 * token-major tensors into head-major pool buffers (the single-GPU stand-in
 * for the Ulysses all-to-all), the attention kernels run on the pool, and the
 * results are copied back.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *     16-byte aligned. The library never allocates or frees device memory and
 *     keeps no pointer after a call returns.
 *   - Layouts: q, out, dout, dq: [S, Hq, d]; k, v, dk, dv: [S, Hkv, d]
 *     (row-major, token-major). lse: [Hq, S] fp32, natural log.
 *   - dtype: UPIPE_BF16 (inputs/outputs bf16, fp32 accumulation) or
 *     UPIPE_FP32 (all fp32). lse is always fp32.
 *   - Supported: d in {64, 128}; Hq % Hkv == 0; head_chunk divides Hq and
 *     either divides G = Hq/Hkv or is a multiple of it; causal in {0, 1};
 *     1 <= S and S*d < 2^31.
 *   - stream: a hipStream_t (NULL = the null stream). All work is enqueued on
 *     it and the call returns without synchronising.
 *   - Errors: every argument is validated on the host before anything is
 *     enqueued. On failure the call returns a negative upipe_status, enqueues
 *     and writes nothing, and upipe_last_error() describes the problem. A
 *     failed kernel launch returns UPIPE_EHIP.
 *   - Determinism: results are bit-identical across head_chunk values and
 *     across repeated calls (fixed key-tile order, no floating-point atomics).
 *   - Outputs (out, out_lo, lse, dq, dk, dv) and the workspace must not
 *     overlap each other or any input.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef UPIPE_ATTN_H
#define UPIPE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { UPIPE_BF16 = 0, UPIPE_FP32 = 1 } upipe_dtype;

typedef enum {
  UPIPE_OK = 0,
  UPIPE_EINVAL = -1,        /* bad argument (null pointer, bad shape, bad head_chunk) */
  UPIPE_EUNSUPPORTED = -2,  /* valid but not supported (head dim, dtype, size) */
  UPIPE_EWORKSPACE = -3,    /* workspace smaller than the *_workspace_bytes value */
  UPIPE_EHIP = -4           /* a HIP runtime call or kernel launch failed */
} upipe_status;

/*
 * Bytes of the fixed buffer pool that upipe_attn_fwd needs (the buffers that
 * every head chunk reuses: the chunk's q and out rows, head-major, and its
 * kv head(s); for bf16 the v head is held transposed in blocks of 64 keys,
 * padded to a multiple of 64 positions). Returns 0 and sets
 * upipe_last_error() on invalid arguments.
 */
size_t upipe_attn_fwd_workspace_bytes(int64_t S, int Hq, int Hkv, int d,
                                      int head_chunk, int dtype);

/*
 * Bytes of the fixed buffer pool that upipe_attn_bwd needs: the chunk's q, dout
 * and dq rows, its kv head(s), the per-row D = <dout, out> and lse*log2(e)
 * terms, and -- only
 * when head_chunk < G, so that one kv head's gradient is summed over several
 * chunks -- fp32 dk/dv accumulators for one kv head.
 * Returns 0 and sets upipe_last_error() on invalid arguments.
 */
size_t upipe_attn_bwd_workspace_bytes(int64_t S, int Hq, int Hkv, int d,
                                      int head_chunk, int dtype);

/*
 * Forward. Reads q, k, v; writes out and lse (every element). Runs the head
 * chunks in ascending head order on `stream`, each through the same workspace.
 *
 * out_lo (bf16 only; may be NULL): receives, element by element, the bf16
 * rounding residual of out, bf16(o - out) where o is the fp32 result, same
 * layout as out. Handing it to upipe_attn_bwd lets the backward form
 * D = <dout, o> from o to about 16 significant bits instead of 8. That
 * matters for rows whose softmax is peaked (every causal row near the start
 * of the sequence): there dP_ij - D_i cancels and a D taken from the rounded
 * out alone can lose most of the gradient's accuracy. Ignored for fp32.
 */
int upipe_attn_fwd(const void* q, const void* k, const void* v,
                   void* out, void* out_lo, float* lse,
                   int64_t S, int Hq, int Hkv, int d, int head_chunk,
                   int causal, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward (recompute-based: the probabilities are rebuilt from q, k and the
 * saved lse instead of being stored). Inputs: q, k, v, the forward's out,
 * out_lo (may be NULL: D then comes from out alone) and lse, and the upstream
 * gradient dout. Writes dq, dk, dv (every element; overwritten, not
 * accumulated into):
 *   D_hi  = <dout_hi, out_hi + out_lo_hi>,  P_ij = exp(s_ij - lse_hi)
 *   dS_ij = P_ij (<dout_hi, v_gj> - D_hi)
 *   dq_hi = tau sum_j dS_ij k_gj
 *   dk_gj = tau sum_{h in group g} sum_i dS_ij q_hi
 *   dv_gj = sum_{h in group g} sum_i P_ij dout_hi
 */
int upipe_attn_bwd(const void* q, const void* k, const void* v,
                   const void* out, const void* out_lo, const void* dout,
                   const float* lse,
                   void* dq, void* dk, void* dv,
                   int64_t S, int Hq, int Hkv, int d, int head_chunk,
                   int causal, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed documents (MaxText long-context article: several samples packed into
 * one long sequence need no padding, and blocks that the mask excludes
 * entirely are skipped). The same forward and backward as above, where a
 * position attends only to positions of its own document -- and, when causal,
 * only to itself and earlier positions of it:
 *   A(i) = { j : doc(j) == doc(i) and (j <= i or causal == 0) }
 * replaces the look-back set in every formula above.
 *
 * doc_offsets: DEVICE pointer to n_docs + 1 int32 values
 *   0 = o_0 <= o_1 <= ... <= o_{n_docs} = S, 4-byte aligned; document m holds
 *   positions o_m .. o_{m+1} - 1 (empty documents are allowed). Owned by the
 *   caller and only read, by the kernels, in stream order.
 * n_docs >= 1. One document [0, S] gives results bit-identical to
 *   upipe_attn_fwd / upipe_attn_bwd.
 * Key tiles outside a query tile's documents are never loaded or computed.
 * Errors: a NULL doc_offsets or n_docs < 1 fails as UPIPE_EINVAL before
 *   anything is enqueued. The offsets themselves live on the device and are
 *   not checked: offsets that break the rules above give unspecified results,
 *   but every access still stays inside the caller's tensors and the pool.
 * Workspace: the same sizes as upipe_attn_fwd / upipe_attn_bwd. The backward
 *   must get the same doc_offsets as the forward that produced out and lse.
 */
int upipe_attn_fwd_docs(const void* q, const void* k, const void* v,
                        void* out, void* out_lo, float* lse,
                        int64_t S, int Hq, int Hkv, int d, int head_chunk,
                        int causal, const int32_t* doc_offsets, int n_docs,
                        int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

int upipe_attn_bwd_docs(const void* q, const void* k, const void* v,
                        const void* out, const void* out_lo, const void* dout,
                        const float* lse,
                        void* dq, void* dk, void* dv,
                        int64_t S, int Hq, int Hkv, int d, int head_chunk,
                        int causal, const int32_t* doc_offsets, int n_docs,
                        int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The head-chunk plan, for inspection (host only, no device work). Fills up to
 * max_chunks entries; entry c describes chunk c:
 *   q_head0[c]  first query head of the chunk (it covers head_chunk heads)
 *   kv_head0[c] first kv head the chunk reads
 *   n_kv[c]     number of kv heads the chunk reads
 *   flags[c]    bit 0: the chunk must (re)load its kv heads into the pool;
 *               bit 1: first chunk that touches kv_head0 (dk/dv start at 0);
 *               bit 2: last chunk that touches kv_head0 (dk/dv are final).
 * Returns the number of chunks (Hq / head_chunk), or a negative upipe_status.
 */
int upipe_attn_plan(int Hq, int Hkv, int head_chunk, int max_chunks,
                    int32_t* q_head0, int32_t* kv_head0, int32_t* n_kv,
                    int32_t* flags);

/*
 * Kernel timing for measurement. While enabled, every kernel the library
 * enqueues is bracketed by a pair of HIP events recorded on the launch stream
 * itself. upipe_profile_read() waits for the recorded events, adds their
 * elapsed times into per-kernel totals, and copies up to max_kernels entries:
 * names[i] (static strings), launches[i], total_ms[i]. Returns the number of
 * kernel kinds seen since the last reset (host only; the totals are shared by
 * all threads and guarded by a lock). upipe_profile_reset() drops all totals
 * and events.
 */
int upipe_profile_enable(int on);
int upipe_profile_read(int max_kernels, const char** names, int64_t* launches, double* total_ms);
void upipe_profile_reset(void);
/* Non-blocking: how many kernels bracketed since the last read/reset have
 * finished, and (if `total` is not NULL) how many were bracketed. Lets a
 * caller report progress of a long asynchronous call as kernels complete. */
int upipe_profile_completed(int* total);

/* Message for the last failed call on this thread ("" if none). Valid until
 * the next call into the library on the same thread. */
const char* upipe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* UPIPE_ATTN_H */
