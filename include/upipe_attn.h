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
 * Quiz answer on U-Pipe). Peak device memory is therefore set by head_chunk,
 * not by Hq. It grows with head_chunk, with one exception: a chunk that holds
 * a whole kv group needs no fp32 dK/dV accumulators, so at Hq/Hkv = 2 in bf16
 * the backward pool is smaller at head_chunk 2 than at 1. Per chunk: the chunk's heads are copied from the caller's
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
 *     1 <= S, S*d < 2^31 and every tensor below 2^48 bytes.
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
 * Bytes of one workspace that serves both upipe_attn_fwd and upipe_attn_bwd
 * (called one after the other, as in training): the larger of the two values
 * above. This is the size of the fixed buffer pool of the chunked method
 * (talk summary, Chapters: heads processed in batches reuse one buffer); it
 * rises strictly with head_chunk and does not depend on Hq beyond that.
 * Returns 0 and sets upipe_last_error() on invalid arguments.
 */
size_t upipe_attn_workspace_bytes(int64_t S, int Hq, int Hkv, int d,
                                  int head_chunk, int dtype);

/*
 * The chunk-size trade-off (talk summary, Chapters: the chunk-size chapter;
 * talk digest, Plan: pick the chunk from the memory left): returns the
 * largest valid head_chunk whose workspace (upipe_attn_workspace_bytes) fits
 * in budget_bytes -- larger chunks take fewer, wider launches and more
 * memory. Every valid head_chunk is considered (pools are not monotone in
 * head_chunk, see above). Host only. Returns UPIPE_EWORKSPACE if no valid
 * head_chunk fits, or another negative status for invalid arguments.
 */
int upipe_attn_pick_head_chunk(int64_t S, int Hq, int Hkv, int d, int dtype,
                               size_t budget_bytes);

/*
 * Forward. Reads q, k, v; writes out and lse (every element). Runs the head
 * chunks in ascending head order on `stream`, each through the same workspace.
 *
 * out_lo (bf16 only; may be NULL): receives, element by element, the bf16
 * rounding residual of out, bf16(o - out) where o is the fp32 result, same
 * layout as out (so it costs one more [S, Hq, d] bf16 tensor of caller
 * memory, e.g. 10 GiB at S = 5,242,880, Hq = 8, d = 128). Handing it to upipe_attn_bwd lets the backward form
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
 * Forward that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, results and errors as upipe_attn_fwd,
 * bit for bit, without the workspace: the fixed buffer pool lives in a
 * static device array of UPIPE_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU
 * holds from the library's first call on it until the process ends. The
 * forward's pool needs nothing cleared between calls (every byte a kernel
 * reads is written earlier in the same call).
 *   - Limit: upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, head_chunk, dtype)
 *     must not exceed UPIPE_NOALLOC_SCRATCH_BYTES (about 65,000 tokens at
 *     Hkv = head_chunk = 1, d = 128, bf16); larger problems fail with
 *     UPIPE_EWORKSPACE before anything is enqueued.
 *   - The current device (hipSetDevice) must be the one that owns the tensors
 *     and the stream: its copy of the array is used.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams, other threads) race on it and must be
 *     serialized by the caller. Calls in stream order are safe.
 *   - No hipMalloc, hipFree or allocating library call is made; the array's
 *     address is looked up once per device (hipGetSymbolAddress).
 */
#define UPIPE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int upipe_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                           void* out, void* out_lo, float* lse,
                           int64_t S, int Hq, int Hkv, int d, int head_chunk,
                           int causal, int dtype, void* stream);

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
 * Fused deterministic backward ("Road to 5 Million Tokens" talk summary,
 * Chapters: the activation-checkpointing chapter -- the backward rebuilds what
 * the forward did not keep; this call rebuilds the scores once per (row
 * block, key tile) pair instead of twice). The same inputs, outputs and
 * formulas as upipe_attn_bwd, from one kv-major kernel that also forms dq:
 * five products per pair instead of seven. dq is summed in a fixed order (per
 * XCD of the device: key tiles in ascending order, each adding after the one
 * before it; then the XCDs' partial sums in ascending order), so repeated
 * calls, and calls with any head_chunk, give bit-identical dq, dk, dv. The
 * values differ from upipe_attn_bwd's by rounding only (another summation
 * order).
 * Limits: bf16 (dtype implied), d = 128, (S + 32) * 512 < 2^32; no document
 *   masks. Other shapes fail with UPIPE_EUNSUPPORTED before anything is
 *   enqueued.
 * max_polls: the longest any wait for another workgroup may poll (0 selects
 *   2^20, seconds). If a wait runs out -- it cannot while the device runs the
 *   call's kernels, but the limit guarantees that every kernel ends -- every
 *   dq value of the chunk is written as NaN instead; dk, dv are then
 *   unspecified. Nothing else changes.
 * Workspace: upipe_attn_bwd_fused_workspace_bytes(); beyond the
 *   upipe_attn_bwd pool it holds eight fp32 dq partial sums of head_chunk
 *   heads (8 * head_chunk * S * d * 4 bytes: 4 GiB per head at S = 1,048,576).
 *   Calls that share a workspace must be serialized (stream order is enough).
 * Returns 0 when everything was enqueued on `stream`; the result of a wait
 * that gave up shows only in dq, as above.
 */
size_t upipe_attn_bwd_fused_workspace_bytes(int64_t S, int Hq, int Hkv, int d,
                                            int head_chunk);

int upipe_attn_bwd_fused(const void* q, const void* k, const void* v,
                         const void* out, const void* out_lo, const void* dout,
                         const float* lse,
                         void* dq, void* dk, void* dv,
                         int64_t S, int Hq, int Hkv, int d, int head_chunk,
                         int causal, int max_polls,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * bf16 GEMM with fp32 accumulation on the MFMA units (the projections around
 * the chunked attention use it; exported so it can be checked on its own):
 *   C[M, N] = A[M, K] B[K, N]   (accumulate != 0, fp32 C only: C += A B)
 * Each operand is described by its contiguous index -- K if *_kmajor != 0
 * (A stored [M][K], B stored [N][K] as a torch Linear weight), else M or N
 * (A stored [K][M], B stored [K][N]) -- and
 *   element (c, o) at ptr + (c / blk) * blk_stride + o * ld + (c % blk),
 * c the contiguous index, o the other one; blk <= 0 means one block (a plain
 * row-major matrix), blk > 0 (a power of two >= 8) lets the contiguous index
 * run in blocks (a head-major [heads][S][d] buffer read as one
 * [S][heads * d] matrix). C is
 *   C[m, n] at c + (n / c_blk) * c_blk_stride + m * ldc + (n % c_blk),
 * bf16 (c_dtype = UPIPE_BF16, rounded to nearest even) or fp32.
 * Requirements: K a multiple of 64; N a multiple of 8; an M- (N-)contiguous
 * operand needs M (N) a multiple of 8; every ld and block stride a multiple
 * of 8 elements, every block length a power of two >= 8; pointers 16-byte
 * aligned; M, N >= 1.
 * Device pointers, owned by the caller; the extents the layouts reach must lie
 * inside the caller's buffers (not checkable here: plain pointers). Errors as
 * for the attention calls; the work is enqueued on `stream`.
 */
int upipe_gemm_bf16(const void* a, int64_t lda, int64_t a_blk, int64_t a_blk_stride, int a_kmajor,
                    const void* b, int64_t ldb, int64_t b_blk, int64_t b_blk_stride, int b_kmajor,
                    void* c, int64_t ldc, int64_t c_blk, int64_t c_blk_stride, int c_dtype,
                    int accumulate, int M, int N, int K, void* stream);

/*
 * Attention block, forward, chunked around the heads (talk summary,
 * Chapters: in the Q&A the head batching is said to target the layer's Q, K
 * and V, full-sequence tensors; the chapter on processing heads in batches).
 * Per head chunk, in ascending head order, through one fixed pool:
 *   q_h = x Wq_h^T, k_g = x Wk_g^T, v_g = x Wv_g^T    (rounded to bf16)
 *   o_h = causal GQA attention of the chunk's heads   (as upipe_attn_fwd)
 *   y  += o_h Wo_h^T, one head at a time, in fp32
 * so no q, k, v or o of all heads over the whole sequence is ever formed.
 *   x   [S, Dm] bf16, the layer input (token-major)
 *   wq  [Hq*d, Dm], wk, wv [Hkv*d, Dm], wo [Dm, Hq*d] bf16, torch Linear
 *       layout [out_features, in_features], no bias; head h owns rows
 *       h*d .. h*d+d-1 of wq and columns h*d .. of wo, kv head g rows g*d ..
 *       of wk and wv (GQA: q head h reads kv head h / (Hq/Hkv))
 *   y   [S, Dm] fp32, written (not accumulated into)
 *   out [S, Hq, d] bf16 or NULL: the attention output, kept only if given
 *   lse [Hq, S] fp32, natural log, as upipe_attn_fwd
 * Dm a multiple of 64; d in {64, 128}; head_chunk as for upipe_attn_fwd. y,
 * out and lse are bit-identical across head_chunk. Workspace:
 * upipe_attn_block_fwd_workspace_bytes (the chunk's q and o rows, its kv
 * heads' k, v and transposed v rows); it rises with head_chunk only.
 */
size_t upipe_attn_block_fwd_workspace_bytes(int64_t S, int Dm, int Hq, int Hkv, int d,
                                            int head_chunk);
int upipe_attn_block_fwd(const void* x, const void* wq, const void* wk, const void* wv,
                         const void* wo, float* y, void* out, float* lse,
                         int64_t S, int Dm, int Hq, int Hkv, int d, int head_chunk,
                         int causal, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention block, backward, chunked around the heads like the forward (the
 * same talk summary passages; the backward runs the chain rule through the
 * forward's steps, each head chunk in ascending order through one pool).
 * Per chunk:
 *   q, k, v of its heads from x again (as the forward)
 *   o: the caller's `out` rows, or (out == NULL) the chunk's attention
 *      forward run again (the recomputation of activation checkpointing)
 *   dO_h = dy Wo_h;  dWo_h = dy^T o_h
 *   dq_h, dk_g, dv_g: the attention backward (as upipe_attn_bwd)
 *   dWq_h = dq_h^T x;  dWk_g = dk_g^T x;  dWv_g = dv_g^T x
 *   dx  += dq_h Wq_h (the chunk's heads of each kv group, in head order),
 *          then dk_g Wk_g + dv_g Wv_g once group g's dk, dv are complete
 *   x, wq, wk, wv, wo as upipe_attn_block_fwd; dy [S, Dm] bf16, the gradient
 *       of y
 *   out [S, Hq, d] bf16 and lse [Hq, S] fp32 from upipe_attn_block_fwd, or
 *       out = NULL (lse is then not read and may be NULL)
 *   dx [S, Dm], dwq [Hq*d, Dm], dwk, dwv [Hkv*d, Dm], dwo [Dm, Hq*d] fp32,
 *       written (not accumulated into)
 * q, k, v, o, dO, dq, dk and dv are bf16 in the pool; the weight gradients
 * sum over tokens in one fixed order (64-token steps, the last one zero
 * padded). Results are bit-identical across head_chunk. Workspace:
 * upipe_attn_block_bwd_workspace_bytes(..., recompute) with recompute = 1 for
 * out == NULL (it adds the transposed v, o's rounding residual and the lse
 * rows); it rises with head_chunk only. Errors as upipe_attn_block_fwd; lse
 * NULL with out given is UPIPE_EINVAL.
 */
size_t upipe_attn_block_bwd_workspace_bytes(int64_t S, int Dm, int Hq, int Hkv, int d,
                                            int head_chunk, int recompute);
int upipe_attn_block_bwd(const void* x, const void* wq, const void* wk, const void* wv,
                         const void* wo, const void* dy, const void* out, const float* lse,
                         float* dx, float* dwq, float* dwk, float* dwv, float* dwo,
                         int64_t S, int Dm, int Hq, int Hkv, int d, int head_chunk,
                         int causal, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sequence-tiled cross-entropy over the vocabulary (talk summary, Chapters:
 * the sequence-tiling chapter -- the loss is computed in pieces along the
 * sequence so that the [S, V] logits never exist at once). Tiles of `tile`
 * tokens go in ascending order through one bounded buffer of tile x V fp32
 * logits (plus tile x V bf16 gradient rows when gradients are asked for):
 *   z_i    = W h_i,  lse_i = ln sum_j exp(z_ij)
 *   loss_i = lse_i - z_i[label_i]                     (0 if label_i < 0)
 *   G_ij   = grad_scale * (exp(z_ij - lse_i) - [j == label_i])   (bf16)
 *   dh_i   = sum_j G_ij W_j,   dw_j = sum_i G_ij h_i  (tile by tile, in order)
 *   h      [S, Dm] bf16 (final hidden states), w [V, Dm] bf16 (torch Linear
 *          layout), labels [S] int32 (negative: ignored; a label >= V is an
 *          error the host cannot see: that token's loss is NaN and, with
 *          gradients, so are its dh row and all of dw; nothing is read out
 *          of bounds)
 *   loss   [S] fp32, natural log
 *   dh     [S, Dm] bf16 or NULL; dw [V, Dm] fp32 or NULL (written, not
 *          accumulated into); both NULL: forward only (no gradient buffer)
 * Dm a multiple of 64, V a multiple of 8, tile a multiple of 64. Results are
 * deterministic (fixed reduction and accumulation orders). Workspace:
 * upipe_ce_loss_workspace_bytes(S, Dm, V, tile, with_grad), independent of S.
 */
size_t upipe_ce_loss_workspace_bytes(int64_t S, int Dm, int V, int tile, int with_grad);
int upipe_ce_loss_tiled(const void* h, const void* w, const int32_t* labels, float* loss,
                        void* dh, float* dw, int64_t S, int Dm, int V, int tile,
                        float grad_scale, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Sequence-tiled SwiGLU MLP (talk summary, Chapters: the sequence-tiling
 * chapter -- the MLP is computed in pieces along the sequence so that its
 * [S, F] intermediates never exist at once). Tiles of `tile` tokens, in
 * ascending order, through one bounded buffer of [tile, F] gate, up and
 * activation rows:
 *   g = x Wg^T, u = x Wu^T  (bf16),  a = silu(g) * u  (bf16),  y = a Wd^T
 *   x, y [S, Dm] bf16; wg, wu [F, Dm], wd [Dm, F] bf16 (torch Linear layout)
 * The backward recomputes each tile's g, u, a from x, then
 *   da = dy Wd,  du = da * silu(g),  dg = da * u * silu'(g)   (dg, du bf16)
 *   dx = dg Wg + du Wu   (fp32, written per tile)
 *   dwg = sum over tiles dg^T x,  dwu = ... du^T x,  dwd = ... dy^T a   (fp32,
 *   tiles in order: deterministic; written, not accumulated into)
 * Dm, F and tile multiples of 64. Workspace: upipe_mlp_workspace_bytes
 * (independent of S).
 */
size_t upipe_mlp_workspace_bytes(int64_t S, int Dm, int F, int tile, int with_grad);
int upipe_mlp_tiled_fwd(const void* x, const void* wg, const void* wu, const void* wd, void* y,
                        int64_t S, int Dm, int F, int tile,
                        void* workspace, size_t workspace_bytes, void* stream);
int upipe_mlp_tiled_bwd(const void* x, const void* wg, const void* wu, const void* wd,
                        const void* dy, float* dx, float* dwg, float* dwu, float* dwd,
                        int64_t S, int Dm, int F, int tile,
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
