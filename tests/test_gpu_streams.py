"""Every entry point runs its work on the stream it is given.

Each call is made twice: once on torch's default stream, and once on a
separate, non-blocking stream (default priority) that is first held up by a
bounded spin kernel and then produces the call's inputs by copying them. A
kernel that the library launched on any other stream would run while that
stream is still spinning, read the copies before they are written, and give
different results; on the given stream it sees the copies, so both calls must
agree bit for bit.
"""

import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import bit_equal
from long_context_attention_upipe_amd.workloads import custom, make_block_inputs, make_inputs

pytestmark = pytest.mark.gpu

SPIN = 50_000_000  # cycles of torch's spin kernel: tens of milliseconds


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _both(fn, *inputs):
    """fn(*inputs) on the default stream, then on a held-up side stream from
    copies made there; returns both results (tuples of tensors)."""
    ref = fn(*inputs)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN)
        copies = [t.clone() for t in inputs]
        got = fn(*copies)
    s.synchronize()
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got, what):
    for i, (a, b) in enumerate(zip(ref, got)):
        assert bit_equal(a, b), f"{what}: output {i} differs on the side stream"


def test_attention_forward_backward_and_fused_on_the_given_stream():
    dev = _dev()
    w = custom(3000, 4, 1, 128, "bf16", seed=77, dout_scaled=True)
    q, k, v, do = (t.to(dev) for t in make_inputs(w, device="cpu"))
    print("\n  attention S=3000 Hq=4 Hkv=1 d=128 on a side stream", flush=True)

    def fn(q, k, v, do):
        out, lse, lo = up.attention_forward(q, k, v, head_chunk=2)
        dq, dk, dv = up.attention_backward(q, k, v, out, do, lse, lo, head_chunk=2)
        fq, fk, fv = up.attention_backward_fused(q, k, v, out, do, lse, lo, head_chunk=2)
        return out, lse, lo, dq, dk, dv, fq, fk, fv

    _same(*_both(fn, q, k, v, do), "attention")


def test_packed_documents_and_noalloc_forward_on_the_given_stream():
    dev = _dev()
    w = custom(2000, 4, 2, 64, "bf16", seed=78, dout_scaled=True)
    q, k, v, do = (t.to(dev) for t in make_inputs(w, device="cpu"))
    offs = torch.tensor([0, 1, 700, 700, 1333, 2000], dtype=torch.int32, device=dev)
    print("\n  documents and the no-allocation forward on a side stream", flush=True)

    def fn(q, k, v, do, offs):
        out, lse, lo = up.attention_forward(q, k, v, head_chunk=2, doc_offsets=offs)
        dq, dk, dv = up.attention_backward(q, k, v, out, do, lse, lo, head_chunk=2, doc_offsets=offs)
        out2 = torch.empty_like(q)
        lo2 = torch.empty_like(q)
        lse2 = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
        up.upipe_attn_fwd_noalloc(q, k, v, out2, lo2, lse2, 1, True)
        return out, lse, lo, dq, dk, dv, out2, lse2, lo2

    _same(*_both(fn, q, k, v, do, offs), "documents / no-allocation forward")


def test_gemm_loss_and_mlp_on_the_given_stream():
    dev = _dev()
    g = torch.Generator(device="cpu").manual_seed(79)
    S, Dm, V, F, tile = 700, 256, 1000, 512, 256
    a = torch.randn((S, Dm), generator=g).to(torch.bfloat16).to(dev)
    b = (torch.randn((V, Dm), generator=g) / 16).to(torch.bfloat16).to(dev)
    labels = torch.randint(0, V, (S,), generator=g, dtype=torch.int32).to(dev)
    wg, wu = ((torch.randn((F, Dm), generator=g) / 16).to(torch.bfloat16).to(dev) for _ in range(2))
    wd = (torch.randn((Dm, F), generator=g) / 22).to(torch.bfloat16).to(dev)
    dy = (torch.randn((S, Dm), generator=g) / S).to(torch.bfloat16).to(dev)
    print("\n  gemm, tiled loss and tiled MLP on a side stream", flush=True)

    def fn(a, b, labels, wg, wu, wd, dy):
        c = torch.empty((S, V), dtype=torch.float32, device=dev)
        up.upipe_gemm_bf16(a, {"ld": Dm, "kmajor": 1}, b, {"ld": Dm, "kmajor": 1}, c, {"ld": V}, S, V, Dm)
        ws = torch.empty(up.upipe_ce_loss_workspace_bytes(S, Dm, V, tile, True), dtype=torch.uint8, device=dev)
        loss = torch.empty((S,), device=dev)
        dh = torch.empty_like(a)
        dw = torch.empty((V, Dm), device=dev)
        up.upipe_ce_loss_tiled(a, b, labels, loss, dh, dw, tile, 1.0 / S, ws)
        wsm = torch.empty(up.upipe_mlp_workspace_bytes(S, Dm, F, tile, True), dtype=torch.uint8, device=dev)
        y = torch.empty_like(a)
        up.upipe_mlp_tiled_fwd(a, wg, wu, wd, y, tile, wsm)
        dx = torch.empty((S, Dm), device=dev)
        dwg, dwu = torch.empty((F, Dm), device=dev), torch.empty((F, Dm), device=dev)
        dwd = torch.empty((Dm, F), device=dev)
        up.upipe_mlp_tiled_bwd(a, wg, wu, wd, dy, dx, dwg, dwu, dwd, tile, wsm)
        return c, loss, dh, dw, y, dx, dwg, dwu, dwd

    _same(*_both(fn, a, b, labels, wg, wu, wd, dy), "gemm / loss / mlp")


def test_attention_block_on_the_given_stream():
    dev = _dev()
    S, Dm, Hq, Hkv, d = 1500, 256, 4, 2, 64
    x, wq, wk, wv, wo = make_block_inputs(S, Dm, Hq, Hkv, d, seed=80, device=dev)
    dy = torch.randn((S, Dm), generator=torch.Generator(device="cpu").manual_seed(81)).to(torch.bfloat16).to(dev)
    print("\n  attention block forward and backward on a side stream", flush=True)

    def fn(x, wq, wk, wv, wo, dy):
        ws = torch.empty(up.upipe_attn_block_fwd_workspace_bytes(S, Dm, Hq, Hkv, d, 2), dtype=torch.uint8,
                         device=dev)
        y = torch.empty((S, Dm), dtype=torch.float32, device=dev)
        out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((Hq, S), dtype=torch.float32, device=dev)
        up.upipe_attn_block_fwd(x, wq, wk, wv, wo, y, out, lse, Hq, Hkv, 2, True, ws)
        wsb = torch.empty(up.upipe_attn_block_bwd_workspace_bytes(S, Dm, Hq, Hkv, d, 2, True), dtype=torch.uint8,
                          device=dev)
        grads = [torch.empty(t.shape, dtype=torch.float32, device=dev) for t in (x, wq, wk, wv, wo)]
        up.upipe_attn_block_bwd(x, wq, wk, wv, wo, dy, None, None, *grads, Hq, Hkv, 2, True, wsb)
        return (y, out, lse, *grads)

    _same(*_both(fn, x, wq, wk, wv, wo, dy), "attention block")
