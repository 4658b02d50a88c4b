"""UPipe causal GQA attention for MI355X (gfx950).

The compute path is the HIP library ``libupipe_attn.so`` behind the C ABI in
``include/upipe_attn.h``; this package only binds it (``_lib``) and adds thin
helpers that let torch allocate the outputs and the fixed buffer pool.
"""

from ._lib import (  # noqa: F401
    NOALLOC_SCRATCH_BYTES,
    UPIPE_BF16,
    UPIPE_FP32,
    UpipeError,
    dtype_code,
    upipe_attn_block_bwd,
    upipe_attn_block_bwd_workspace_bytes,
    upipe_attn_block_fwd,
    upipe_attn_block_fwd_workspace_bytes,
    upipe_attn_bwd,
    upipe_attn_bwd_docs,
    upipe_attn_bwd_fused,
    upipe_attn_bwd_fused_workspace_bytes,
    upipe_attn_bwd_workspace_bytes,
    upipe_attn_fwd,
    upipe_attn_fwd_docs,
    upipe_attn_fwd_noalloc,
    upipe_attn_fwd_workspace_bytes,
    upipe_attn_pick_head_chunk,
    upipe_attn_plan,
    upipe_attn_workspace_bytes,
    upipe_ce_loss_tiled,
    upipe_ce_loss_workspace_bytes,
    upipe_gemm_bf16,
    upipe_mlp_tiled_bwd,
    upipe_mlp_tiled_fwd,
    upipe_mlp_workspace_bytes,
    upipe_last_error,
    upipe_profile_completed,
    upipe_profile_enable,
    upipe_profile_read,
    upipe_profile_reset,
)


def workspace(S, Hq, Hkv, d, head_chunk, dtype, device="cuda", which="both"):
    """Allocate the fixed buffer pool (uint8) for the forward, backward or both."""
    import torch

    code = dtype_code(dtype) if not isinstance(dtype, int) else dtype
    sizes = []
    if which in ("fwd", "both"):
        sizes.append(upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, head_chunk, code))
    if which in ("bwd", "both"):
        sizes.append(upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, head_chunk, code))
    return torch.empty(max(sizes), dtype=torch.uint8, device=device)


def attention_forward(q, k, v, head_chunk=1, causal=True, ws=None, stream=None, residual=True, doc_offsets=None):
    """(out, lse, out_lo) of attention over [S,Hq,d] / [S,Hkv,d] device tensors.

    out_lo is out's bf16 rounding residual (None for fp32 or residual=False);
    pass it to attention_backward for an accurate D = <dout, out>.
    doc_offsets (int32 [n_docs + 1] on the device, 0 .. S) packs documents:
    each position then attends only within its own document."""
    import torch

    S, Hq, d = q.shape
    Hkv = k.shape[1]
    out = torch.empty_like(q)
    out_lo = torch.empty_like(q) if (residual and q.dtype == torch.bfloat16) else None
    lse = torch.empty((Hq, S), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(S, Hq, Hkv, d, head_chunk, q.dtype, q.device, "fwd")
    if doc_offsets is None:
        upipe_attn_fwd(q, k, v, out, out_lo, lse, head_chunk, causal, ws, stream)
    else:
        upipe_attn_fwd_docs(q, k, v, out, out_lo, lse, head_chunk, causal, doc_offsets, ws, stream)
    return out, lse, out_lo


def attention_backward(q, k, v, out, dout, lse, out_lo=None, head_chunk=1, causal=True, ws=None, stream=None,
                       doc_offsets=None):
    """dq, dk, dv of attention given the forward's out, lse (and out_lo), and
    the forward's doc_offsets if it had them."""
    import torch

    S, Hq, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if ws is None:
        ws = workspace(S, Hq, Hkv, d, head_chunk, q.dtype, q.device, "bwd")
    if doc_offsets is None:
        upipe_attn_bwd(q, k, v, out, out_lo, dout, lse, dq, dk, dv, head_chunk, causal, ws, stream)
    else:
        upipe_attn_bwd_docs(q, k, v, out, out_lo, dout, lse, dq, dk, dv, head_chunk, causal, doc_offsets, ws,
                            stream)
    return dq, dk, dv


def attention_backward_fused(q, k, v, out, dout, lse, out_lo=None, head_chunk=1, causal=True, ws=None,
                             stream=None, max_polls=0):
    """dq, dk, dv from the fused deterministic backward (bf16, d = 128)."""
    import torch

    S, Hq, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if ws is None:
        ws = torch.empty(upipe_attn_bwd_fused_workspace_bytes(S, Hq, Hkv, d, head_chunk), dtype=torch.uint8,
                         device=q.device)
    upipe_attn_bwd_fused(q, k, v, out, out_lo, dout, lse, dq, dk, dv, head_chunk, causal, ws, max_polls, stream)
    return dq, dk, dv


def wait_reporting(what, device=None, interval=10.0, prefix="[upipe]", log=None):
    """Block until enqueued work is done, printing a line (to stderr, or
    through ``log``) as the library's kernels finish, at most every
    ``interval`` seconds.

    Kernels are counted only while profiling is on (``upipe_profile_enable``);
    with it off this is a plain device synchronize. Multi-million-token calls
    run for minutes, and the line shows they are progressing."""
    import sys
    import time

    import torch

    seen, last = 0, time.perf_counter()
    while True:
        done, total = upipe_profile_completed()
        now = time.perf_counter()
        if done > seen and (done == total or now - last > interval):
            line = f"{prefix} {what}: {done}/{total} kernels finished"
            if log is None:
                print(line, file=sys.stderr, flush=True)
            else:
                log(line)
            seen, last = done, now
        if done == total:
            break
        time.sleep(0.002)
    torch.cuda.synchronize(device)
