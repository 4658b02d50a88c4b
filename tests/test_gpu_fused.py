"""The fused deterministic backward (upipe_attn_bwd_fused) through the C ABI
against the fp64 oracle, on full tensors: ragged lengths, several key tiles
per XCD queue (so workgroups wait for each other's dQ additions), two kv
heads, causal and not, every head_chunk. Its results must be bit-identical
across head_chunk and across repeated calls, and a wait whose poll limit runs
out (forced from the host with a limit of one poll) must show as NaN in dQ
and leave later calls unaffected. Every case prints its shape first.
"""

import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import assert_close, bit_equal, f64, grad_scale
from long_context_attention_upipe_amd.workloads import custom, make_inputs
from oracle.attention import attention_backward

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _forward(q, k, v, causal):
    out, lse, out_lo = up.attention_forward(q, k, v, head_chunk=1, causal=causal)
    return out, lse, out_lo


def _fused(q, k, v, out, do, lse, out_lo, hc, causal, max_polls=0):
    dq, dk, dv = up.attention_backward_fused(q, k, v, out, do, lse, out_lo, head_chunk=hc, causal=causal,
                                             max_polls=max_polls)
    torch.cuda.synchronize()
    return dict(dq=dq, dk=dk, dv=dv)


def _case(w, hcs, causal=True):
    dev = _dev()
    print(f"\n  fused case S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} causal={causal} hcs={hcs}", flush=True)
    q, k, v, do = make_inputs(w, device="cpu")
    rdq, rdk, rdv = attention_backward(f64(q), f64(k), f64(v), f64(do), causal=causal)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse, out_lo = _forward(qd, kd, vd, causal)
    gs = grad_scale(w)
    first = None
    for hc in hcs:
        print(f"   head_chunk={hc}", flush=True)
        r = _fused(qd, kd, vd, out, dod, lse, out_lo, hc, causal)
        assert_close("dq", f64(r["dq"]), rdq, w.dtype, grad_scale=gs, per_item=True)
        assert_close("dk", f64(r["dk"]), rdk, w.dtype, grad_scale=gs, per_item=True)
        assert_close("dv", f64(r["dv"]), rdv, w.dtype, grad_scale=gs, per_item=True)
        if first is None:
            first = r
            again = _fused(qd, kd, vd, out, dod, lse, out_lo, hc, causal)
            for name in r:
                assert bit_equal(r[name], again[name]), f"{name}: a repeated call differs"
        else:
            for name in r:
                assert bit_equal(r[name], first[name]), f"{name} differs between head_chunk {hcs[0]} and {hc}"


@pytest.mark.parametrize("S", [1, 2, 31, 127, 128, 129, 300, 1000])
def test_fused_ragged_lengths(S):
    _case(custom(S, 4, 1, 128, "bf16", seed=400 + S, dout_scaled=True), (1, 2, 4))


def test_fused_many_tiles_per_queue():
    """65 key tiles: 8 or 9 per XCD queue, each adding after the one before."""
    _case(custom(8269, 4, 1, 128, "bf16", seed=41, dout_scaled=True), (1, 4))


def test_fused_two_kv_heads_every_chunk_size():
    """Hkv = 2: head_chunk 1 and 2 carry dK/dV across chunks in fp32; 8 runs
    both kv heads in one launch (tickets alternate between them)."""
    _case(custom(1500, 8, 2, 128, "bf16", seed=43, dout_scaled=True), (1, 2, 4, 8))


def test_fused_non_causal():
    _case(custom(2100, 4, 1, 128, "bf16", seed=47, dout_scaled=True), (1, 4), causal=False)


def test_fused_close_to_two_kernel_backward():
    """Same gradients as the two-kernel backward up to rounding order."""
    dev = _dev()
    w = custom(3000, 4, 1, 128, "bf16", seed=53, dout_scaled=True)
    print(f"\n  fused vs two-kernel S={w.S}", flush=True)
    q, k, v, do = (t.to(dev) for t in make_inputs(w, device="cpu"))
    out, lse, out_lo = _forward(q, k, v, True)
    r = _fused(q, k, v, out, do, lse, out_lo, 1, True)
    dq, dk, dv = up.attention_backward(q, k, v, out, do, lse, out_lo, head_chunk=1, causal=True)
    torch.cuda.synchronize()
    gs = grad_scale(w)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(name, f64(r[name]), f64(ref), w.dtype, grad_scale=gs, per_item=True)


def test_fused_wait_limit_poisons_dq_and_later_calls_recover():
    """max_polls = 1: a wait that finds the previous tile's additions still
    missing gives up at once. Either no wait had to wait (then the result is
    the normal one, bit for bit) or dQ is NaN everywhere; dK and dV are
    unspecified then. The next call with the default limit is exact again."""
    dev = _dev()
    w = custom(8269, 4, 1, 128, "bf16", seed=59, dout_scaled=True)
    print(f"\n  forced give-up S={w.S}", flush=True)
    q, k, v, do = (t.to(dev) for t in make_inputs(w, device="cpu"))
    out, lse, out_lo = _forward(q, k, v, True)
    normal = _fused(q, k, v, out, do, lse, out_lo, 1, True)
    forced = _fused(q, k, v, out, do, lse, out_lo, 1, True, max_polls=1)
    n_nan = int(torch.isnan(forced["dq"].float()).sum())
    print(f"   NaN in dq: {n_nan} of {forced['dq'].numel()}", flush=True)
    if n_nan:
        assert n_nan == forced["dq"].numel(), "a wait gave up, so every dq value must be NaN"
    else:
        for name in normal:
            assert bit_equal(forced[name], normal[name]), name
    after = _fused(q, k, v, out, do, lse, out_lo, 1, True)
    for name in normal:
        assert bit_equal(after[name], normal[name]), f"{name}: the call after the forced one differs"


def test_fused_rejects_unsupported_shapes_before_launch():
    dev = _dev()
    q = torch.zeros((64, 4, 64), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((64, 1, 64), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((4, 64), dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    with pytest.raises(up.UpipeError, match="d = 128"):
        up.upipe_attn_bwd_fused(q, k, k, q, None, q, lse, torch.empty_like(q), torch.empty_like(k),
                                torch.empty_like(k), 1, 1, ws)
    q32 = q.float()
    with pytest.raises(up.UpipeError):
        up.upipe_attn_bwd_fused(q32, k.float(), k.float(), q32, None, q32, lse, torch.empty_like(q32),
                                torch.empty_like(k.float()), torch.empty_like(k.float()), 1, 1, ws)
