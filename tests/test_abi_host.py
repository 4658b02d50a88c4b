"""C ABI checks that need no GPU: the library loads and exports every
declared symbol, the head-chunk planner, pool sizes, and argument validation
(which runs on the host before anything is enqueued)."""

import ctypes
import os
import re

import pytest

from long_context_attention_upipe_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "upipe_attn.h")

FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: validation fails first


def declared_functions():
    with open(HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(upipe_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = L.lib()
    names = declared_functions()
    assert {"upipe_attn_fwd", "upipe_attn_bwd", "upipe_attn_fwd_workspace_bytes",
            "upipe_attn_bwd_workspace_bytes", "upipe_attn_plan", "upipe_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"


@pytest.mark.parametrize("Hq,Hkv,hc", [(4, 1, 1), (4, 1, 2), (4, 1, 4), (8, 1, 8), (8, 2, 1), (8, 2, 2),
                                       (8, 2, 4), (8, 2, 8), (4, 4, 1), (4, 4, 4), (6, 2, 3)])
def test_plan_covers_heads_in_order(Hq, Hkv, hc):
    plan = L.upipe_attn_plan(Hq, Hkv, hc)
    G = Hq // Hkv
    assert len(plan) == Hq // hc
    assert [c["q_head0"] for c in plan] == list(range(0, Hq, hc))
    seen_first, seen_last = set(), set()
    prev_kv = None
    for c in plan:
        heads = range(c["q_head0"], c["q_head0"] + hc)
        kvs = sorted({h // G for h in heads})
        assert c["kv_head0"] == kvs[0] and c["n_kv"] == len(kvs)
        assert c["load_kv"] == (c["kv_head0"] != prev_kv)
        prev_kv = c["kv_head0"]
        if c["first_for_kv"]:
            assert c["q_head0"] % G == 0
            seen_first.add(c["kv_head0"])
        if c["last_for_kv"]:
            assert (c["q_head0"] + hc) % G == 0
            seen_last.add(c["kv_head0"])
    assert seen_first == seen_last == set(range(0, Hkv, max(1, hc // G)))


@pytest.mark.parametrize("S,Hq,Hkv,d,hcs", [(131072, 4, 1, 128, (1, 2, 4)), (5242880, 8, 1, 128, (1, 2, 4, 8)),
                                            (1024, 4, 4, 64, (1, 4)), (1000, 8, 2, 128, (1, 2, 4, 8))])
@pytest.mark.parametrize("dtype", [0, 1])
def test_pool_grows_strictly_with_head_chunk(S, Hq, Hkv, d, hcs, dtype):
    fwd = [L.upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, hc, dtype) for hc in hcs]
    bwd = [L.upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, hc, dtype) for hc in hcs]
    assert all(a < b for a, b in zip(fwd, fwd[1:])), fwd
    assert all(a < b for a, b in zip(bwd, bwd[1:])), bwd
    es = 2 if dtype == 0 else 4
    U = S * d * es
    # the forward pool holds the chunk's q and out rows and its kv heads; bf16 v
    # heads are stored transposed with rows padded to a multiple of 64 positions
    Uv = ((S + 63) // 64 * 64 if dtype == 0 else S) * d * es
    for hc, n in zip(hcs, fwd):
        nkv = max(1, hc // (Hq // Hkv))
        assert 2 * hc * U + nkv * (U + Uv) <= n < 2 * hc * U + nkv * (U + Uv) + 4096


def test_pool_at_5m_tokens_matches_plan():
    # the largest share: S = 5,242,880, Hq = 8, Hkv = 1, d = 128, bf16
    gib = 1 << 30
    sizes = [L.upipe_attn_bwd_workspace_bytes(5242880, 8, 1, 128, hc, 0) / gib for hc in (1, 2, 4, 8)]
    U = 5242880 * 128 * 2 / gib
    # q, dO, dq rows of the chunk; k, v; D and lse*log2(e) per row; fp32 dk/dv when a group spans chunks
    expect = [3 * hc * U + 2 * U + 2 * hc * 5242880 * 4 / gib + (4 * U if hc < 8 else 0) for hc in (1, 2, 4, 8)]
    for got, exp in zip(sizes, expect):
        assert abs(got - exp) < 1e-3


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, out_lo=None, lse=FAKE, S=256, Hq=4, Hkv=1, d=128, hc=1, causal=1,
             dtype=0, ws=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return L.lib().upipe_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["out_lo"], a["lse"], a["S"], a["Hq"], a["Hkv"],
                                  a["d"],
                                  a["hc"], a["causal"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


def _bwd(**kw):
    a = dict(S=256, Hq=4, Hkv=1, d=128, hc=1, causal=1, dtype=0, ws_bytes=1 << 40, dq=FAKE, out_lo=None)
    a.update(kw)
    return L.lib().upipe_attn_bwd(FAKE, FAKE, FAKE, FAKE, a["out_lo"], FAKE, FAKE, a["dq"], FAKE, FAKE, a["S"], a["Hq"],
                                  a["Hkv"],
                                  a["d"], a["hc"], a["causal"], a["dtype"], FAKE, a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(S=0), -1, "S must be"),
    (dict(Hq=4, Hkv=3), -1, "multiple of Hkv"),
    (dict(hc=3), -1, "must divide Hq"),
    (dict(Hq=12, Hkv=2, hc=4), -1, "divide or be a multiple"),
    (dict(causal=2), -1, "causal"),
    (dict(d=96), -2, "head dim"),
    (dict(dtype=7), -2, "dtype"),
    (dict(S=1 << 25), -2, "2^31"),
    (dict(q=None), -1, "q is NULL"),
    (dict(lse=None), -1, "lse is NULL"),
    (dict(out=ctypes.c_void_p(0x10008)), -1, "not 16-byte aligned"),
    (dict(ws_bytes=1024), -3, "workspace too small"),
    (dict(out_lo=ctypes.c_void_p(0x10004)), -1, "out_lo is not 16-byte aligned"),
])
def test_forward_rejects_bad_arguments(kw, status, msg):
    assert _fwd(**kw) == status
    assert msg in L.upipe_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(hc=8), -1, "must divide Hq"),
    (dict(dq=None), -1, "dq is NULL"),
    (dict(ws_bytes=0), -3, "workspace too small"),
    (dict(d=32), -2, "head dim"),
    (dict(out_lo=ctypes.c_void_p(0x10002)), -1, "out_lo is not 16-byte aligned"),
])
def test_backward_rejects_bad_arguments(kw, status, msg):
    assert _bwd(**kw) == status
    assert msg in L.upipe_last_error()


def test_workspace_bytes_reports_errors():
    assert L.lib().upipe_attn_fwd_workspace_bytes(0, 4, 1, 128, 1, 0) == 0
    assert "S must be" in L.upipe_last_error()
    with pytest.raises(L.UpipeError):
        L.upipe_attn_bwd_workspace_bytes(16, 4, 1, 128, 3, 0)
    assert L.upipe_attn_fwd_workspace_bytes(16, 4, 1, 128, 2, 0) > 0
    assert L.upipe_last_error() == ""


def test_plan_rejects_small_table():
    n = 4
    arrs = [(ctypes.c_int32 * 1)() for _ in range(4)]
    assert L.lib().upipe_attn_plan(n, 1, 1, 1, *arrs) == -1
    assert "max_chunks" in L.upipe_last_error()


@pytest.mark.parametrize("name,bad", [
    ("v", {"v": (64, 2, 32)}),
    ("out", {"out": (64, 4, 32)}),
    ("lse", {"lse": (64, 4)}),
    ("dk", {"dk": (64, 1, 64)}),
])
def test_binding_rejects_mismatched_shapes(name, bad):
    """The C ABI takes plain pointers; the binding checks every extent first."""
    import torch

    S, Hq, Hkv, d = 64, 4, 2, 64
    shapes = {"k": (S, Hkv, d), "v": (S, Hkv, d), "out": (S, Hq, d), "lse": (Hq, S), "dk": (S, Hkv, d)}
    shapes.update(bad)
    q = torch.empty(S, Hq, d)
    named = [(n, torch.empty(shp), exp) for n, shp, exp in [
        ("k", shapes["k"], (S, Hkv, d)), ("v", shapes["v"], (S, Hkv, d)), ("out", shapes["out"], (S, Hq, d)),
        ("lse", shapes["lse"], (Hq, S)), ("dk", shapes["dk"], (S, Hkv, d))]]
    with pytest.raises(L.UpipeError, match=f"{name} has shape"):
        L._require_shapes(q, named)
    L._require_shapes(q, [(n, torch.empty(exp), exp) for n, _, exp in named])


def _fwd_docs(offsets=FAKE, n_docs=3, **kw):
    a = dict(S=256, Hq=4, Hkv=1, d=128, hc=1, causal=1, dtype=0, ws_bytes=1 << 40)
    a.update(kw)
    return L.lib().upipe_attn_fwd_docs(FAKE, FAKE, FAKE, FAKE, None, FAKE, a["S"], a["Hq"], a["Hkv"], a["d"], a["hc"],
                                       a["causal"], offsets, n_docs, a["dtype"], FAKE, a["ws_bytes"], None)


def _bwd_docs(offsets=FAKE, n_docs=3, **kw):
    a = dict(S=256, Hq=4, Hkv=1, d=128, hc=1, causal=1, dtype=0, ws_bytes=1 << 40)
    a.update(kw)
    return L.lib().upipe_attn_bwd_docs(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, a["S"], a["Hq"],
                                       a["Hkv"], a["d"], a["hc"], a["causal"], offsets, n_docs, a["dtype"], FAKE,
                                       a["ws_bytes"], None)


@pytest.mark.parametrize("call", [_fwd_docs, _bwd_docs], ids=["fwd", "bwd"])
@pytest.mark.parametrize("kw,status,msg", [
    (dict(offsets=None), -1, "doc_offsets is NULL"),
    (dict(offsets=None, n_docs=0), -1, "doc_offsets is NULL"),
    (dict(n_docs=0), -1, "n_docs must be >= 1"),
    (dict(n_docs=-2), -1, "n_docs must be >= 1"),
    (dict(offsets=ctypes.c_void_p(0x10002)), -1, "not 4-byte aligned"),
    (dict(hc=3), -1, "must divide Hq"),
    (dict(ws_bytes=16), -3, "workspace too small"),
])
def test_document_entry_points_reject_bad_arguments(call, kw, status, msg):
    assert call(**kw) == status
    assert msg in L.upipe_last_error()


@pytest.mark.parametrize("offsets,msg", [
    ([0, 10, 64], None),
    ([0, 0, 64, 64], None),
    ([0, 64], None),
    ([1, 10, 64], "rise"),
    ([0, 10, 63], "rise"),
    ([0, 30, 20, 64], "rise"),
    ([64], "at least two"),
])
def test_binding_checks_document_offsets(offsets, msg):
    """The library reads the offsets on the device only, so the binding checks
    their values (here on CPU tensors; the same code runs on device tensors)."""
    import torch

    q = torch.empty(64, 4, 32)
    t = torch.tensor(offsets, dtype=torch.int32)
    if msg is None:
        assert L._require_docs(q, t) == len(offsets) - 1
    else:
        with pytest.raises(L.UpipeError, match=msg):
            L._require_docs(q, t)
    with pytest.raises(L.UpipeError, match="int32"):
        L._require_docs(q, t.long())


@pytest.mark.parametrize("S,Hq,Hkv,d,hcs", [(131072, 4, 1, 128, (1, 2, 4)), (5242880, 8, 1, 128, (1, 2, 4, 8)),
                                            (1024, 4, 4, 64, (1, 4)), (1000, 8, 2, 128, (1, 2, 4, 8))])
@pytest.mark.parametrize("dtype", [0, 1])
def test_workspace_bytes_is_the_larger_pool(S, Hq, Hkv, d, hcs, dtype):
    """One workspace for the forward and the backward of a training step."""
    prev = 0
    for hc in hcs:
        both = L.upipe_attn_workspace_bytes(S, Hq, Hkv, d, hc, dtype)
        assert both == max(L.upipe_attn_fwd_workspace_bytes(S, Hq, Hkv, d, hc, dtype),
                           L.upipe_attn_bwd_workspace_bytes(S, Hq, Hkv, d, hc, dtype))
        assert both > prev
        prev = both
    assert L.lib().upipe_attn_workspace_bytes(S, Hq, Hkv, d, 3, dtype) == 0
    assert "head_chunk" in L.upipe_last_error()


def test_pick_head_chunk_takes_the_largest_pool_that_fits():
    S, Hq, Hkv, d = 5242880, 8, 1, 128
    sizes = {hc: L.upipe_attn_workspace_bytes(S, Hq, Hkv, d, hc, 0) for hc in (1, 2, 4, 8)}
    for hc, n in sizes.items():
        assert L.upipe_attn_pick_head_chunk(S, Hq, Hkv, d, 0, n) == hc
        if hc > 1:
            assert L.upipe_attn_pick_head_chunk(S, Hq, Hkv, d, 0, n - 1) == hc // 2
    assert L.upipe_attn_pick_head_chunk(S, Hq, Hkv, d, 0, 1 << 50) == 8
    # Hq = 6, Hkv = 2 (G = 3): the valid chunks are 1, 3, 6, never 2
    sizes6 = {hc: L.upipe_attn_workspace_bytes(4096, 6, 2, 64, hc, 0) for hc in (1, 3, 6)}
    assert L.upipe_attn_pick_head_chunk(4096, 6, 2, 64, 0, sizes6[3] + 100) == 3
    assert L.upipe_attn_pick_head_chunk(4096, 6, 2, 64, 0, sizes6[6] - 1) == 3
    with pytest.raises(L.UpipeError, match="no head_chunk fits"):
        L.upipe_attn_pick_head_chunk(S, Hq, Hkv, d, 0, sizes[1] - 1)
    with pytest.raises(L.UpipeError, match="head dim"):
        L.upipe_attn_pick_head_chunk(S, Hq, Hkv, 96, 0, 1 << 50)


def test_size_limits_at_the_boundary():
    """S*d < 2^31 is the only length limit: copy kernels index tokens with 64
    bits, so a total vector count at or above 2^32 (where a 32-bit grid-stride
    index would wrap) is accepted. Host-only: sizes are computed, nothing runs."""
    d = 128
    assert L.upipe_attn_fwd_workspace_bytes((1 << 24) - 1, 1, 1, d, 1, 0) > 0  # S*d = 2^31 - 128
    assert L.lib().upipe_attn_fwd_workspace_bytes(1 << 24, 1, 1, d, 1, 0) == 0  # S*d = 2^31
    assert "2^31" in L.upipe_last_error()
    # q with Hq = head_chunk = 64 at S = 4,193,000: 2^32 - 1.1e6 sixteen-byte vectors per pack
    S, H = 4193000, 64
    assert S * H * d * 2 // 16 > (1 << 32) - (1 << 21)
    assert L.upipe_attn_fwd_workspace_bytes(S, H, 1, d, H, 0) > 0
    # and past 2^32 vectors
    assert S * 128 * d * 2 // 16 > (1 << 32)
    assert L.upipe_attn_bwd_workspace_bytes(S, 128, 1, d, 128, 0) > 0


def test_noalloc_forward_host_checks():
    """upipe_attn_fwd_noalloc validates like the workspace forward and rejects
    a pool larger than its static array before touching any device."""
    lib = L.lib()
    args = lambda S, hc=1, d=128: (FAKE, FAKE, FAKE, FAKE, None, FAKE, S, 4, 1, d, hc, 1, 0, None)  # noqa: E731
    assert lib.upipe_attn_fwd_noalloc(*args(70000)) == -3
    assert "static scratch" in L.upipe_last_error()
    assert L.upipe_attn_fwd_workspace_bytes(70000, 4, 1, 128, 1, 0) > L.NOALLOC_SCRATCH_BYTES
    assert lib.upipe_attn_fwd_noalloc(*args(1000, hc=3)) == -1
    assert "must divide Hq" in L.upipe_last_error()
    assert lib.upipe_attn_fwd_noalloc(*args(1000, d=96)) == -2
    with open(HEADER) as f:
        assert "#define UPIPE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in f.read()
    assert L.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_block_and_gemm_host_checks():
    lib = L.lib()
    S, Dm, Hq, Hkv, d = 4096, 512, 4, 1, 128
    sizes = [L.upipe_attn_block_fwd_workspace_bytes(S, Dm, Hq, Hkv, d, hc) for hc in (1, 2, 4)]
    assert sizes[0] < sizes[1] < sizes[2]
    U = S * d * 2
    assert sizes[0] >= 2 * U + 3 * U  # q, o; k, v, transposed v
    assert lib.upipe_attn_block_fwd_workspace_bytes(S, 100, Hq, Hkv, d, 1) == 0
    assert "multiple of 64" in L.upipe_last_error()
    blk = lambda **kw: lib.upipe_attn_block_fwd(*(kw.get(n, FAKE) for n in ("x", "wq", "wk", "wv", "wo", "y")),  # noqa: E731
                                                kw.get("out"), kw.get("lse", FAKE), S, kw.get("Dm", Dm), Hq, Hkv, d,
                                                kw.get("hc", 1), 1, FAKE, kw.get("ws", 1 << 40), None)
    assert blk(wo=None) == -1 and "wo is NULL" in L.upipe_last_error()
    assert blk(Dm=96) == -2
    assert blk(hc=3) == -1
    assert blk(ws=16) == -3
    assert blk(out=ctypes.c_void_p(0x10002)) == -1 and "out is not 16-byte aligned" in L.upipe_last_error()
    # the backward's pool: more than the forward's, rises with head_chunk,
    # and recomputing o adds the transposed v, o's residual and lse rows
    bsz = [L.upipe_attn_block_bwd_workspace_bytes(S, Dm, Hq, Hkv, d, hc, True) for hc in (1, 2, 4)]
    assert bsz[0] < bsz[1] < bsz[2] and bsz[0] > sizes[0]
    kept = L.upipe_attn_block_bwd_workspace_bytes(S, Dm, Hq, Hkv, d, 1, False)
    assert bsz[0] - kept >= 2 * U + S * 4  # transposed v, o residual, lse rows
    assert lib.upipe_attn_block_bwd_workspace_bytes(S, 100, Hq, Hkv, d, 1, 1) == 0
    names = ("x", "wq", "wk", "wv", "wo", "dy")
    grads = ("dx", "dwq", "dwk", "dwv", "dwo")
    bwd = lambda **kw: lib.upipe_attn_block_bwd(*(kw.get(n, FAKE) for n in names), kw.get("out"),  # noqa: E731
                                                kw.get("lse"), *(kw.get(n, FAKE) for n in grads), S,
                                                kw.get("Dm", Dm), Hq, Hkv, d, kw.get("hc", 1), 1, FAKE,
                                                kw.get("ws", 1 << 40), None)
    assert bwd(dy=None) == -1 and "dy is NULL" in L.upipe_last_error()
    assert bwd(dwv=None) == -1 and "dwv is NULL" in L.upipe_last_error()
    assert bwd(out=FAKE) == -1 and "lse is NULL" in L.upipe_last_error()
    assert bwd(Dm=96) == -2
    assert bwd(hc=3) == -1
    assert bwd(ws=16) == -3 and "workspace too small" in L.upipe_last_error()
    # recomputing o needs the larger pool: a pool sized without it is refused
    assert bwd(ws=kept) == -3
    gemm = lambda M=64, N=64, K=64, lda=64, a_km=1, c_dtype=1, acc=0, a=FAKE: lib.upipe_gemm_bf16(  # noqa: E731
        a, lda, 0, 0, a_km, FAKE, K, 0, 0, 1, FAKE, N, 0, 0, c_dtype, acc, M, N, K, None)
    assert gemm(K=100) == -2 and "multiple of 64" in L.upipe_last_error()
    assert gemm(N=60) == -2
    assert gemm(acc=1, c_dtype=0) == -1 and "fp32" in L.upipe_last_error()
    assert gemm(lda=60) == -1
    assert gemm(M=60, a_km=0, lda=64) == -1 and "multiple of 8" in L.upipe_last_error()
    assert gemm(a=None) == -1 and "a is NULL" in L.upipe_last_error()
    assert gemm(M=0) == -1


def test_tiled_loss_host_checks():
    lib = L.lib()
    # the buffer is one tile's logits (+ its gradient rows), whatever S is
    a = L.upipe_ce_loss_workspace_bytes(1 << 20, 4096, 128256, 2048, True)
    b = L.upipe_ce_loss_workspace_bytes(5 << 20, 4096, 128256, 2048, True)
    assert a == b
    Vp = (128256 + 63) // 64 * 64
    assert a >= 2048 * Vp * (4 + 2)
    assert L.upipe_ce_loss_workspace_bytes(1 << 20, 4096, 128256, 2048, False) < a
    call = lambda **kw: lib.upipe_ce_loss_tiled(  # noqa: E731
        kw.get("h", FAKE), FAKE, FAKE, FAKE, None, None, kw.get("S", 1000), kw.get("Dm", 128), kw.get("V", 1000),
        kw.get("tile", 128), 1.0, FAKE, kw.get("ws", 1 << 40), None)
    assert call(V=1001) == -2 and "multiple of 8" in L.upipe_last_error()
    assert call(tile=100) == -1 and "tile" in L.upipe_last_error()
    assert call(Dm=100) == -2
    assert call(h=None) == -1 and "h is NULL" in L.upipe_last_error()
    assert call(ws=16) == -3
    assert call(S=0) == -1


def test_tiled_mlp_host_checks():
    lib = L.lib()
    a = L.upipe_mlp_workspace_bytes(1 << 20, 4096, 14336, 4096, True)
    assert a == L.upipe_mlp_workspace_bytes(5 << 20, 4096, 14336, 4096, True)  # independent of S
    assert a >= 4096 * 14336 * (3 * 2 + 4)
    assert L.upipe_mlp_workspace_bytes(1 << 20, 4096, 14336, 4096, False) < a
    fwd = lambda **kw: lib.upipe_mlp_tiled_fwd(kw.get("x", FAKE), FAKE, FAKE, FAKE, FAKE, kw.get("S", 1000),  # noqa: E731
                                               kw.get("Dm", 128), kw.get("F", 256), kw.get("tile", 128), FAKE,
                                               kw.get("ws", 1 << 40), None)
    assert fwd(F=100) == -2 and "multiple of 64" in L.upipe_last_error()
    assert fwd(tile=96) == -1
    assert fwd(x=None) == -1 and "x is NULL" in L.upipe_last_error()
    assert fwd(ws=16) == -3
    assert lib.upipe_mlp_tiled_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1000, 128, 256, 128, FAKE,
                                   1 << 40, None) == -1
    assert "dx is NULL" in L.upipe_last_error()


def test_fused_backward_host_checks():
    lib = L.lib()
    S = 1 << 20
    n1 = L.upipe_attn_bwd_fused_workspace_bytes(S, 4, 1, 128, 1)
    n4 = L.upipe_attn_bwd_fused_workspace_bytes(S, 4, 1, 128, 4)
    assert n1 < n4
    # the two-kernel pool without its packed dq, plus eight fp32 dq partials of the chunk's heads
    two_kernel = L.upipe_attn_bwd_workspace_bytes(S, 4, 1, 128, 1, L.UPIPE_BF16)
    assert n1 >= two_kernel - S * 128 * 2 + 8 * S * 128 * 4
    assert lib.upipe_attn_bwd_fused_workspace_bytes(1000, 4, 1, 64, 1) == 0
    assert "d = 128" in L.upipe_last_error()
    assert lib.upipe_attn_bwd_fused_workspace_bytes(8388576, 1, 1, 128, 1) == 0
    assert "2^32" in L.upipe_last_error()
    assert lib.upipe_attn_bwd_fused_workspace_bytes(8388575, 1, 1, 128, 1) > 0

    def call(**kw):
        a = dict(dq=FAKE, S=1000, Hq=4, Hkv=1, d=128, hc=1, causal=1, polls=0, ws=1 << 40)
        a.update(kw)
        return lib.upipe_attn_bwd_fused(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, a["dq"], FAKE, FAKE, a["S"],
                                        a["Hq"], a["Hkv"], a["d"], a["hc"], a["causal"], a["polls"], FAKE, a["ws"],
                                        None)

    assert call(d=64) == -2 and "d = 128" in L.upipe_last_error()
    assert call(dq=None) == -1 and "dq is NULL" in L.upipe_last_error()
    assert call(polls=-1) == -1 and "max_polls" in L.upipe_last_error()
    assert call(ws=16) == -3 and "workspace too small" in L.upipe_last_error()
    assert call(hc=3) == -1 and "must divide Hq" in L.upipe_last_error()
    assert call(causal=2) == -1


def _c_declarations():
    """(name, return type, [parameter types]) of every function the header
    declares, comments removed, whitespace normalised."""
    with open(HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    out = []
    for ret, name, params in re.findall(r"([A-Za-z_][\w\s\*]*?)\b(upipe_\w+)\s*\(([^;{]*?)\)\s*;", src, flags=re.S):
        ps = [" ".join(p.split()) for p in params.split(",")] if params.strip() not in ("", "void") else []
        # drop the parameter name: the type is everything before the last identifier
        types = [re.sub(r"\s*\b\w+$", "", p) for p in ps]
        out.append((name, " ".join(ret.split()), types))
    return out


def _ctype_matches(c_type, ct):
    if c_type.endswith("*"):
        # any pointer: void*, POINTER(...) or a char* string
        return ct in (ctypes.c_void_p, ctypes.c_char_p) or (isinstance(ct, type) and issubclass(ct, ctypes._Pointer))
    plain = {"int64_t": ctypes.c_int64, "int": ctypes.c_int, "size_t": ctypes.c_size_t, "float": ctypes.c_float,
             "double": ctypes.c_double}
    return ct is plain[c_type]


def test_bindings_match_the_header_parameter_by_parameter():
    """Every declared function is bound with as many arguments as the header
    gives it, each of the same kind (pointer, int64_t, int, size_t, float),
    and the same kind of result: a binding that drifted from the header would
    pass its arguments in the wrong registers without any error."""
    lib = L.lib()
    decls = _c_declarations()
    assert len(decls) == len(declared_functions())
    for name, ret, params in decls:
        fn = getattr(lib, name)
        assert fn.argtypes is not None, f"{name}: no argtypes bound"
        assert len(fn.argtypes) == len(params), f"{name}: {len(fn.argtypes)} bound arguments, header has {len(params)}"
        for i, (c_type, ct) in enumerate(zip(params, fn.argtypes)):
            assert _ctype_matches(c_type, ct), f"{name} argument {i}: header {c_type!r}, bound {ct}"
        if ret == "void":
            assert fn.restype is None, name
        else:
            assert _ctype_matches(ret, fn.restype), f"{name} result: header {ret!r}, bound {fn.restype}"
