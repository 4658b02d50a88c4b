"""ctypes binding of libupipe_attn.so (C ABI declared in include/upipe_attn.h).

Argument marshalling only: torch supplies device memory (``data_ptr``) and the
stream handle; every step of the computation runs in the library's HIP
kernels. There is no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_NAME = "libupipe_attn.so"
_HERE = os.path.dirname(os.path.abspath(__file__))
# UPIPE_ATTN_LIBRARY may name another build of the same library (same ABI).
LIB_PATH = os.environ.get("UPIPE_ATTN_LIBRARY") or os.path.join(_HERE, _LIB_NAME)

UPIPE_BF16 = 0
UPIPE_FP32 = 1
STATUS = {0: "UPIPE_OK", -1: "UPIPE_EINVAL", -2: "UPIPE_EUNSUPPORTED", -3: "UPIPE_EWORKSPACE", -4: "UPIPE_EHIP"}

_lib = None


class UpipeError(RuntimeError):
    """A negative status from the library, with its message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, sz, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    L.upipe_attn_fwd_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32]
    L.upipe_attn_fwd_workspace_bytes.restype = sz
    L.upipe_attn_bwd_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32]
    L.upipe_attn_bwd_workspace_bytes.restype = sz
    L.upipe_attn_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32]
    L.upipe_attn_workspace_bytes.restype = sz
    L.upipe_attn_pick_head_chunk.argtypes = [i64, i32, i32, i32, i32, sz]
    L.upipe_attn_pick_head_chunk.restype = i32
    L.upipe_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    L.upipe_attn_fwd.restype = i32
    L.upipe_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, vp, sz,
                                 vp]
    L.upipe_attn_bwd.restype = i32
    L.upipe_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, vp]
    L.upipe_attn_fwd_noalloc.restype = i32
    L.upipe_gemm_bf16.argtypes = [vp, i64, i64, i64, i32, vp, i64, i64, i64, i32, vp, i64, i64, i64, i32, i32, i32,
                                  i32, i32, vp]
    L.upipe_gemm_bf16.restype = i32
    L.upipe_attn_block_fwd_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32]
    L.upipe_attn_block_fwd_workspace_bytes.restype = sz
    L.upipe_attn_block_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    L.upipe_attn_block_fwd.restype = i32
    L.upipe_attn_block_bwd_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32, i32]
    L.upipe_attn_block_bwd_workspace_bytes.restype = sz
    L.upipe_attn_block_bwd.argtypes = [vp] * 13 + [i64, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    L.upipe_attn_block_bwd.restype = i32
    L.upipe_ce_loss_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    L.upipe_ce_loss_workspace_bytes.restype = sz
    L.upipe_ce_loss_tiled.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, ctypes.c_float, vp, sz, vp]
    L.upipe_ce_loss_tiled.restype = i32
    L.upipe_mlp_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    L.upipe_mlp_workspace_bytes.restype = sz
    L.upipe_mlp_tiled_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, vp, sz, vp]
    L.upipe_mlp_tiled_fwd.restype = i32
    L.upipe_mlp_tiled_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, vp, sz, vp]
    L.upipe_mlp_tiled_bwd.restype = i32
    # The packed-document and fused-backward entry points are bound when the
    # loaded build has them (UPIPE_ATTN_LIBRARY may name an older build);
    # calling them on a build without them raises AttributeError.
    if hasattr(L, "upipe_attn_fwd_docs"):
        L.upipe_attn_fwd_docs.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, vp, i32, i32, vp,
                                          sz, vp]
        L.upipe_attn_fwd_docs.restype = i32
        L.upipe_attn_bwd_docs.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, vp,
                                          i32, i32, vp, sz, vp]
        L.upipe_attn_bwd_docs.restype = i32
    if hasattr(L, "upipe_attn_bwd_fused"):
        L.upipe_attn_bwd_fused_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
        L.upipe_attn_bwd_fused_workspace_bytes.restype = sz
        L.upipe_attn_bwd_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, i32,
                                           vp, sz, vp]
        L.upipe_attn_bwd_fused.restype = i32
    p32 = ctypes.POINTER(ctypes.c_int32)
    L.upipe_attn_plan.argtypes = [i32, i32, i32, i32, p32, p32, p32, p32]
    L.upipe_attn_plan.restype = i32
    L.upipe_profile_enable.argtypes = [i32]
    L.upipe_profile_enable.restype = i32
    L.upipe_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_double)]
    L.upipe_profile_read.restype = i32
    L.upipe_profile_completed.argtypes = [ctypes.POINTER(ctypes.c_int)]
    L.upipe_profile_completed.restype = i32
    L.upipe_profile_reset.argtypes = []
    L.upipe_profile_reset.restype = None
    L.upipe_last_error.argtypes = []
    L.upipe_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def upipe_last_error() -> str:
    return lib().upipe_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise UpipeError(status, upipe_last_error())


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return UPIPE_BF16
    if dt == torch.float32:
        return UPIPE_FP32
    raise UpipeError(-2, f"unsupported dtype {dt}")


def upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, head_chunk, dtype) -> int:
    n = lib().upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, head_chunk, dtype)
    if n == 0:
        raise UpipeError(-1, upipe_last_error())
    return n


def upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, head_chunk, dtype) -> int:
    n = lib().upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, head_chunk, dtype)
    if n == 0:
        raise UpipeError(-1, upipe_last_error())
    return n


def upipe_attn_bwd_fused_workspace_bytes(S, Hq, Hkv, d, head_chunk) -> int:
    """Bytes of the fused backward's pool (bf16, d = 128)."""
    n = lib().upipe_attn_bwd_fused_workspace_bytes(S, Hq, Hkv, d, head_chunk)
    if n == 0:
        raise UpipeError(-2, upipe_last_error())
    return n


def upipe_attn_workspace_bytes(S, Hq, Hkv, d, head_chunk, dtype) -> int:
    """Bytes of one workspace serving both the forward and the backward."""
    n = lib().upipe_attn_workspace_bytes(S, Hq, Hkv, d, head_chunk, dtype)
    if n == 0:
        raise UpipeError(-1, upipe_last_error())
    return n


def upipe_attn_pick_head_chunk(S, Hq, Hkv, d, dtype, budget_bytes) -> int:
    """Largest valid head_chunk whose workspace fits in ``budget_bytes``."""
    rc = lib().upipe_attn_pick_head_chunk(S, Hq, Hkv, d, dtype, int(budget_bytes))
    if rc < 0:
        raise UpipeError(rc, upipe_last_error())
    return rc


def upipe_attn_plan(Hq, Hkv, head_chunk):
    """The head-chunk plan as a list of dicts (host only)."""
    n = max(1, Hq)
    arrs = [(ctypes.c_int32 * n)() for _ in range(4)]
    rc = lib().upipe_attn_plan(Hq, Hkv, head_chunk, n, *arrs)
    if rc < 0:
        raise UpipeError(rc, upipe_last_error())
    return [dict(q_head0=arrs[0][i], kv_head0=arrs[1][i], n_kv=arrs[2][i],
                 load_kv=bool(arrs[3][i] & 1), first_for_kv=bool(arrs[3][i] & 2),
                 last_for_kv=bool(arrs[3][i] & 4)) for i in range(rc)]


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(None if t is None else t.data_ptr())


def _shape(q, k):
    if q.dim() != 3 or k.dim() != 3:
        raise UpipeError(-1, "q and k must be [S, H, d]")
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    return S, Hq, Hkv, d


def _require(ts, dt):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise UpipeError(-1, "tensors must be contiguous device tensors")
        if t.dtype != dt:
            raise UpipeError(-1, f"dtype mismatch: {t.dtype} vs {dt}")


def _require_shapes(q, named):
    """The library sees plain pointers, so every buffer's extent is checked
    here: a wrong shape would otherwise become an out-of-bounds access."""
    S, Hq, d = q.shape
    dev = q.device
    for name, t, shape in named:
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape):
            raise UpipeError(-1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.device != dev:
            raise UpipeError(-1, f"{name} is on {t.device}, q on {dev}")


def upipe_attn_fwd(q, k, v, out, out_lo, lse, head_chunk, causal, workspace, stream=None) -> None:
    """Enqueue the forward on ``stream`` (default: torch's current stream).
    ``out_lo`` (bf16, like ``out``, or None) receives out's rounding residual."""
    S, Hq, Hkv, d = _shape(q, k)
    _require((q, k, v, out) + ((out_lo,) if out_lo is not None else ()), q.dtype)
    _require((lse,), torch.float32)
    _require((workspace,), torch.uint8)
    _require_shapes(q, [("k", k, (S, Hkv, d)), ("v", v, (S, Hkv, d)), ("out", out, (S, Hq, d)),
                        ("out_lo", out_lo, (S, Hq, d)), ("lse", lse, (Hq, S)),
                        ("workspace", workspace, (workspace.numel(),))])
    with torch.cuda.device(q.device):
        _check(lib().upipe_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(out_lo), _ptr(lse), S, Hq, Hkv, d,
                                    int(head_chunk), int(causal), dtype_code(q.dtype),
                                    _ptr(workspace), workspace.numel(), _stream_handle(stream)))


# Bytes of the static device array behind upipe_attn_fwd_noalloc (the
# header's UPIPE_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def upipe_attn_fwd_noalloc(q, k, v, out, out_lo, lse, head_chunk, causal, stream=None) -> None:
    """The forward without a workspace: the library's static per-GPU scratch
    array holds the pool, and nothing is allocated. Calls that overlap in time
    on one GPU race on that array; calls in stream order are safe."""
    S, Hq, Hkv, d = _shape(q, k)
    _require((q, k, v, out) + ((out_lo,) if out_lo is not None else ()), q.dtype)
    _require((lse,), torch.float32)
    _require_shapes(q, [("k", k, (S, Hkv, d)), ("v", v, (S, Hkv, d)), ("out", out, (S, Hq, d)),
                        ("out_lo", out_lo, (S, Hq, d)), ("lse", lse, (Hq, S))])
    with torch.cuda.device(q.device):
        _check(lib().upipe_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(out_lo), _ptr(lse), S, Hq,
                                            Hkv, d, int(head_chunk), int(causal), dtype_code(q.dtype),
                                            _stream_handle(stream)))


def upipe_attn_bwd(q, k, v, out, out_lo, dout, lse, dq, dk, dv, head_chunk, causal, workspace, stream=None) -> None:
    """Enqueue the backward on ``stream`` (default: torch's current stream)."""
    S, Hq, Hkv, d = _shape(q, k)
    _require((q, k, v, out, dout, dq, dk, dv) + ((out_lo,) if out_lo is not None else ()), q.dtype)
    _require((lse,), torch.float32)
    _require((workspace,), torch.uint8)
    qs, ks = (S, Hq, d), (S, Hkv, d)
    _require_shapes(q, [("k", k, ks), ("v", v, ks), ("out", out, qs), ("out_lo", out_lo, qs), ("dout", dout, qs),
                        ("lse", lse, (Hq, S)), ("dq", dq, qs), ("dk", dk, ks), ("dv", dv, ks),
                        ("workspace", workspace, (workspace.numel(),))])
    with torch.cuda.device(q.device):
        _check(lib().upipe_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(out_lo), _ptr(dout), _ptr(lse),
                                    _ptr(dq), _ptr(dk), _ptr(dv), S, Hq, Hkv, d,
                                    int(head_chunk), int(causal), dtype_code(q.dtype),
                                    _ptr(workspace), workspace.numel(), _stream_handle(stream)))


def upipe_attn_bwd_fused(q, k, v, out, out_lo, dout, lse, dq, dk, dv, head_chunk, causal, workspace,
                         max_polls=0, stream=None) -> None:
    """Enqueue the fused deterministic backward (bf16, d = 128) on ``stream``.
    ``max_polls`` bounds every wait for another workgroup (0: the library's
    default); a wait that runs out leaves dq all NaN."""
    S, Hq, Hkv, d = _shape(q, k)
    if q.dtype != torch.bfloat16:
        raise UpipeError(-2, f"the fused backward supports bf16 only (got {q.dtype})")
    _require((q, k, v, out, dout, dq, dk, dv) + ((out_lo,) if out_lo is not None else ()), q.dtype)
    _require((lse,), torch.float32)
    _require((workspace,), torch.uint8)
    qs, ks = (S, Hq, d), (S, Hkv, d)
    _require_shapes(q, [("k", k, ks), ("v", v, ks), ("out", out, qs), ("out_lo", out_lo, qs), ("dout", dout, qs),
                        ("lse", lse, (Hq, S)), ("dq", dq, qs), ("dk", dk, ks), ("dv", dv, ks),
                        ("workspace", workspace, (workspace.numel(),))])
    with torch.cuda.device(q.device):
        _check(lib().upipe_attn_bwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(out_lo), _ptr(dout),
                                          _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), S, Hq, Hkv, d,
                                          int(head_chunk), int(causal), int(max_polls),
                                          _ptr(workspace), workspace.numel(), _stream_handle(stream)))


def _require_docs(q, doc_offsets, check_values=True) -> int:
    """Checks the packed-document offsets (int32 [n_docs + 1] on q's device,
    rising from 0 to S) and returns n_docs. The library reads them on the
    device only, so their values are checked here (one device sync; a caller
    that has checked them once may pass check_values=False)."""
    S = q.shape[0]
    t = doc_offsets
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise UpipeError(-1, "doc_offsets must be a contiguous 1-D int32 tensor")
    if t.device != q.device:
        raise UpipeError(-1, f"doc_offsets is on {t.device}, q on {q.device}")
    if t.numel() < 2:
        raise UpipeError(-1, "doc_offsets needs at least two entries (0 and S)")
    if not check_values:
        return t.numel() - 1
    ok = (t[0] == 0) & (t[-1] == S) & (t[1:] >= t[:-1]).all()
    if not bool(ok.item()):
        raise UpipeError(-1, f"doc_offsets must rise (non-strictly) from 0 to S={S}")
    return t.numel() - 1


def upipe_attn_fwd_docs(q, k, v, out, out_lo, lse, head_chunk, causal, doc_offsets, workspace, stream=None,
                        check_offsets=True) -> None:
    """Forward over packed documents (``doc_offsets``: int32 [n_docs + 1] on the device)."""
    S, Hq, Hkv, d = _shape(q, k)
    _require((q, k, v, out) + ((out_lo,) if out_lo is not None else ()), q.dtype)
    _require((lse,), torch.float32)
    _require((workspace,), torch.uint8)
    _require_shapes(q, [("k", k, (S, Hkv, d)), ("v", v, (S, Hkv, d)), ("out", out, (S, Hq, d)),
                        ("out_lo", out_lo, (S, Hq, d)), ("lse", lse, (Hq, S)),
                        ("workspace", workspace, (workspace.numel(),))])
    n_docs = _require_docs(q, doc_offsets, check_offsets)
    with torch.cuda.device(q.device):
        _check(lib().upipe_attn_fwd_docs(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(out_lo), _ptr(lse), S, Hq, Hkv,
                                         d, int(head_chunk), int(causal), _ptr(doc_offsets), n_docs,
                                         dtype_code(q.dtype), _ptr(workspace), workspace.numel(),
                                         _stream_handle(stream)))


def upipe_attn_bwd_docs(q, k, v, out, out_lo, dout, lse, dq, dk, dv, head_chunk, causal, doc_offsets, workspace,
                        stream=None, check_offsets=True) -> None:
    """Backward over packed documents (the same ``doc_offsets`` as the forward)."""
    S, Hq, Hkv, d = _shape(q, k)
    _require((q, k, v, out, dout, dq, dk, dv) + ((out_lo,) if out_lo is not None else ()), q.dtype)
    _require((lse,), torch.float32)
    _require((workspace,), torch.uint8)
    qs, ks = (S, Hq, d), (S, Hkv, d)
    _require_shapes(q, [("k", k, ks), ("v", v, ks), ("out", out, qs), ("out_lo", out_lo, qs), ("dout", dout, qs),
                        ("lse", lse, (Hq, S)), ("dq", dq, qs), ("dk", dk, ks), ("dv", dv, ks),
                        ("workspace", workspace, (workspace.numel(),))])
    n_docs = _require_docs(q, doc_offsets, check_offsets)
    with torch.cuda.device(q.device):
        _check(lib().upipe_attn_bwd_docs(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(out_lo), _ptr(dout), _ptr(lse),
                                         _ptr(dq), _ptr(dk), _ptr(dv), S, Hq, Hkv, d,
                                         int(head_chunk), int(causal), _ptr(doc_offsets), n_docs,
                                         dtype_code(q.dtype), _ptr(workspace), workspace.numel(),
                                         _stream_handle(stream)))


def upipe_profile_enable(on: bool) -> None:
    """Bracket every library kernel launch with HIP events on its stream."""
    lib().upipe_profile_enable(1 if on else 0)


def upipe_profile_reset() -> None:
    lib().upipe_profile_reset()


def upipe_profile_read():
    """{kernel name: (launches, total ms)} since the last reset (waits for the events)."""
    n_max = 16
    names = (ctypes.c_char_p * n_max)()
    launches = (ctypes.c_int64 * n_max)()
    ms = (ctypes.c_double * n_max)()
    n = lib().upipe_profile_read(n_max, names, launches, ms)
    if n < 0:
        raise UpipeError(n, upipe_last_error())
    return {names[i].decode(): (int(launches[i]), float(ms[i])) for i in range(min(n, n_max))}


def upipe_profile_completed():
    """(kernels finished, kernels bracketed) since the last read/reset; non-blocking."""
    total = ctypes.c_int(0)
    done = lib().upipe_profile_completed(ctypes.byref(total))
    return int(done), int(total.value)


def upipe_gemm_bf16(a, a_layout, b, b_layout, c, c_layout, M, N, K, accumulate=False, stream=None) -> None:
    """C[M, N] (+)= A[M, K] B[K, N] on the library's bf16 MFMA GEMM.

    Each layout is a dict: ``ld`` (stride of the non-contiguous index),
    ``kmajor`` (operands: K is the contiguous index), and optionally ``blk`` /
    ``blk_stride`` (the contiguous index runs in blocks). The caller states
    the layout; the library sees plain pointers, so the extent each layout
    reaches is checked here against the tensor's storage."""
    for name, t, lay, outer, dt in (("a", a, a_layout, M, torch.bfloat16), ("b", b, b_layout, N, torch.bfloat16),
                                    ("c", c, c_layout, M, c.dtype)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != dt:
            raise UpipeError(-1, f"{name}: a contiguous {dt} device tensor is required")
        # (contiguous index extent, other index extent)
        if name == "c":
            contig, other = N, M
        elif lay["kmajor"]:
            contig, other = K, outer
        else:
            contig, other = outer, K
        blk = lay.get("blk", 0) or contig
        last = ((contig - 1) // blk) * lay.get("blk_stride", 0) + (other - 1) * lay["ld"] + ((contig - 1) % blk)
        if last >= t.numel():
            raise UpipeError(-1, f"{name}: the layout reaches element {last}, beyond the tensor's {t.numel()}")
    code = UPIPE_FP32 if c.dtype == torch.float32 else UPIPE_BF16
    with torch.cuda.device(a.device):
        _check(lib().upipe_gemm_bf16(_ptr(a), a_layout["ld"], a_layout.get("blk", 0), a_layout.get("blk_stride", 0),
                                     int(a_layout["kmajor"]), _ptr(b), b_layout["ld"], b_layout.get("blk", 0),
                                     b_layout.get("blk_stride", 0), int(b_layout["kmajor"]), _ptr(c),
                                     c_layout["ld"], c_layout.get("blk", 0), c_layout.get("blk_stride", 0), code,
                                     int(bool(accumulate)), M, N, K, _stream_handle(stream)))


def upipe_attn_block_fwd_workspace_bytes(S, Dm, Hq, Hkv, d, head_chunk) -> int:
    n = lib().upipe_attn_block_fwd_workspace_bytes(S, Dm, Hq, Hkv, d, head_chunk)
    if n == 0:
        raise UpipeError(-1, upipe_last_error())
    return n


def upipe_attn_block_fwd(x, wq, wk, wv, wo, y, out, lse, n_q_heads, n_kv_heads, head_chunk, causal, workspace,
                         stream=None) -> None:
    """Attention block forward, chunk by chunk: q, k, v of the chunk's heads
    from x, causal GQA attention, and the chunk's share of y = o Wo^T.
    x [S, Dm] bf16; wq [Hq*d, Dm], wk, wv [Hkv*d, Dm], wo [Dm, Hq*d] bf16
    (torch Linear layout); y [S, Dm] fp32; out [S, Hq, d] bf16 or None;
    lse [Hq, S] fp32."""
    if x.dim() != 2 or wq.dim() != 2:
        raise UpipeError(-1, "x and the weights must be 2-D")
    S, Dm = x.shape
    Hq, Hkv = int(n_q_heads), int(n_kv_heads)
    if wq.shape[0] % Hq:
        raise UpipeError(-1, "wq's rows must be Hq * d")
    d = wq.shape[0] // Hq
    _require((x, wq, wk, wv, wo) + ((out,) if out is not None else ()), torch.bfloat16)
    _require((y, lse), torch.float32)
    _require((workspace,), torch.uint8)
    for name, t, shape in (("wq", wq, (Hq * d, Dm)), ("wk", wk, (Hkv * d, Dm)), ("wv", wv, (Hkv * d, Dm)),
                           ("wo", wo, (Dm, Hq * d)), ("y", y, (S, Dm)), ("out", out, (S, Hq, d)),
                           ("lse", lse, (Hq, S)), ("workspace", workspace, (workspace.numel(),))):
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape):
            raise UpipeError(-1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.device != x.device:
            raise UpipeError(-1, f"{name} is on {t.device}, x on {x.device}")
    with torch.cuda.device(x.device):
        _check(lib().upipe_attn_block_fwd(_ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(y), _ptr(out),
                                          _ptr(lse), S, Dm, Hq, Hkv, d, int(head_chunk), int(causal),
                                          _ptr(workspace), workspace.numel(), _stream_handle(stream)))


def upipe_attn_block_bwd_workspace_bytes(S, Dm, Hq, Hkv, d, head_chunk, recompute=True) -> int:
    n = lib().upipe_attn_block_bwd_workspace_bytes(S, Dm, Hq, Hkv, d, head_chunk, int(bool(recompute)))
    if n == 0:
        raise UpipeError(-1, upipe_last_error())
    return n


def upipe_attn_block_bwd(x, wq, wk, wv, wo, dy, out, lse, dx, dwq, dwk, dwv, dwo, n_q_heads, n_kv_heads, head_chunk,
                         causal, workspace, stream=None) -> None:
    """Attention block backward, chunk by chunk, for the upstream gradient dy
    [S, Dm] bf16 of y: dx [S, Dm] and dwq, dwk, dwv, dwo (the weights'
    shapes) fp32, written. out [S, Hq, d] bf16 and lse [Hq, S] fp32 from the
    forward, or out = None to run the chunk's attention forward again (lse is
    then not read)."""
    if x.dim() != 2 or wq.dim() != 2:
        raise UpipeError(-1, "x and the weights must be 2-D")
    S, Dm = x.shape
    Hq, Hkv = int(n_q_heads), int(n_kv_heads)
    if wq.shape[0] % Hq:
        raise UpipeError(-1, "wq's rows must be Hq * d")
    d = wq.shape[0] // Hq
    _require((x, wq, wk, wv, wo, dy) + ((out,) if out is not None else ()), torch.bfloat16)
    _require((dx, dwq, dwk, dwv, dwo) + ((lse,) if out is not None else ()), torch.float32)
    _require((workspace,), torch.uint8)
    if out is None:
        lse = None
    for name, t, shape in (("wq", wq, (Hq * d, Dm)), ("wk", wk, (Hkv * d, Dm)), ("wv", wv, (Hkv * d, Dm)),
                           ("wo", wo, (Dm, Hq * d)), ("dy", dy, (S, Dm)), ("out", out, (S, Hq, d)),
                           ("lse", lse, (Hq, S)), ("dx", dx, (S, Dm)), ("dwq", dwq, (Hq * d, Dm)),
                           ("dwk", dwk, (Hkv * d, Dm)), ("dwv", dwv, (Hkv * d, Dm)), ("dwo", dwo, (Dm, Hq * d)),
                           ("workspace", workspace, (workspace.numel(),))):
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape):
            raise UpipeError(-1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.device != x.device:
            raise UpipeError(-1, f"{name} is on {t.device}, x on {x.device}")
    with torch.cuda.device(x.device):
        _check(lib().upipe_attn_block_bwd(_ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wo), _ptr(dy), _ptr(out),
                                          _ptr(lse), _ptr(dx), _ptr(dwq), _ptr(dwk), _ptr(dwv), _ptr(dwo), S, Dm,
                                          Hq, Hkv, d, int(head_chunk), int(causal), _ptr(workspace),
                                          workspace.numel(), _stream_handle(stream)))


def upipe_ce_loss_workspace_bytes(S, Dm, V, tile, with_grad=True) -> int:
    n = lib().upipe_ce_loss_workspace_bytes(S, Dm, V, tile, int(bool(with_grad)))
    if n == 0:
        raise UpipeError(-1, upipe_last_error())
    return n


def upipe_ce_loss_tiled(h, w, labels, loss, dh, dw, tile, grad_scale, workspace, stream=None) -> None:
    """Cross-entropy of h [S, Dm] (bf16) against labels [S] (int32, < 0
    ignored) through the vocabulary projection w [V, Dm] (bf16, torch Linear
    layout), one tile of tokens at a time: loss [S] fp32; when given, dh
    [S, Dm] bf16 and dw [V, Dm] fp32 (written, not accumulated into) are the
    gradients of sum(grad_scale * loss)."""
    if h.dim() != 2 or w.dim() != 2:
        raise UpipeError(-1, "h and w must be 2-D")
    S, Dm = h.shape
    V = w.shape[0]
    _require((h, w) + ((dh,) if dh is not None else ()), torch.bfloat16)
    _require((loss,) + ((dw,) if dw is not None else ()), torch.float32)
    _require((labels,), torch.int32)
    _require((workspace,), torch.uint8)
    for name, t, shape in (("w", w, (V, Dm)), ("labels", labels, (S,)), ("loss", loss, (S,)), ("dh", dh, (S, Dm)),
                           ("dw", dw, (V, Dm)), ("workspace", workspace, (workspace.numel(),))):
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape):
            raise UpipeError(-1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.device != h.device:
            raise UpipeError(-1, f"{name} is on {t.device}, h on {h.device}")
    with torch.cuda.device(h.device):
        _check(lib().upipe_ce_loss_tiled(_ptr(h), _ptr(w), _ptr(labels), _ptr(loss), _ptr(dh), _ptr(dw), S, Dm, V,
                                         int(tile), float(grad_scale), _ptr(workspace), workspace.numel(),
                                         _stream_handle(stream)))


def upipe_mlp_workspace_bytes(S, Dm, F, tile, with_grad=True) -> int:
    n = lib().upipe_mlp_workspace_bytes(S, Dm, F, tile, int(bool(with_grad)))
    if n == 0:
        raise UpipeError(-1, upipe_last_error())
    return n


def _mlp_shapes(x, wg, wu, wd, named):
    if x.dim() != 2 or wg.dim() != 2:
        raise UpipeError(-1, "x and the weights must be 2-D")
    S, Dm = x.shape
    F = wg.shape[0]
    for name, t, shape in [("wg", wg, (F, Dm)), ("wu", wu, (F, Dm)), ("wd", wd, (Dm, F))] + named(S, Dm, F):
        if tuple(t.shape) != tuple(shape):
            raise UpipeError(-1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.device != x.device:
            raise UpipeError(-1, f"{name} is on {t.device}, x on {x.device}")
    return S, Dm, F


def upipe_mlp_tiled_fwd(x, wg, wu, wd, y, tile, workspace, stream=None) -> None:
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T, one tile of tokens at a time.
    x [S, Dm], wg, wu [F, Dm], wd [Dm, F] (torch Linear layout), y [S, Dm]:
    all bf16."""
    _require((x, wg, wu, wd, y), torch.bfloat16)
    _require((workspace,), torch.uint8)
    S, Dm, F = _mlp_shapes(x, wg, wu, wd, lambda S, Dm, F: [("y", y, (S, Dm))])
    with torch.cuda.device(x.device):
        _check(lib().upipe_mlp_tiled_fwd(_ptr(x), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(y), S, Dm, F, int(tile),
                                         _ptr(workspace), workspace.numel(), _stream_handle(stream)))


def upipe_mlp_tiled_bwd(x, wg, wu, wd, dy, dx, dwg, dwu, dwd, tile, workspace, stream=None) -> None:
    """Gradients of the tiled SwiGLU MLP given dy [S, Dm] (bf16): dx [S, Dm]
    and dwg, dwu [F, Dm], dwd [Dm, F], all fp32, written (not accumulated
    into). Each tile's activations are recomputed from x."""
    _require((x, wg, wu, wd, dy), torch.bfloat16)
    _require((dx, dwg, dwu, dwd), torch.float32)
    _require((workspace,), torch.uint8)
    S, Dm, F = _mlp_shapes(x, wg, wu, wd, lambda S, Dm, F: [
        ("dy", dy, (S, Dm)), ("dx", dx, (S, Dm)), ("dwg", dwg, (F, Dm)), ("dwu", dwu, (F, Dm)), ("dwd", dwd, (Dm, F))])
    with torch.cuda.device(x.device):
        _check(lib().upipe_mlp_tiled_bwd(_ptr(x), _ptr(wg), _ptr(wu), _ptr(wd), _ptr(dy), _ptr(dx), _ptr(dwg),
                                         _ptr(dwu), _ptr(dwd), S, Dm, F, int(tile), _ptr(workspace),
                                         workspace.numel(), _stream_handle(stream)))
