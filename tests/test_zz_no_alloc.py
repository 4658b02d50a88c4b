"""The forward that allocates nothing (upipe_attn_fwd_noalloc, for callers
that cannot allocate device memory), through the C ABI: bit-identical to the
workspace forward it shares its kernels with, and within the oracle's
tolerance, on two calls in a row on one GPU, the second one smaller (the
static scratch array keeps the first call's contents), with no device memory
allocated by the second call."""

import numpy as np
import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import assert_close, bit_equal, f64
from long_context_attention_upipe_amd.workloads import custom, make_inputs
from oracle.attention import attention_forward

pytestmark = pytest.mark.gpu

CASES = [  # (S, Hq, Hkv, d, head_chunk, dtype, seed): the second is smaller
    (3000, 4, 1, 128, 2, "bf16", 301),
    (777, 4, 2, 64, 1, "bf16", 302),
]


def test_noalloc_forward_two_calls_match_workspace_forward():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    prepared = []
    for S, Hq, Hkv, d, hc, dtype, seed in CASES:
        w = custom(S, Hq, Hkv, d, dtype, seed=seed)
        q, k, v, _ = make_inputs(w, device=dev, need_dout=False)
        ref = up.attention_forward(q, k, v, head_chunk=hc, causal=True)  # the workspace entry point
        got = (torch.empty_like(q), torch.empty((Hq, S), dtype=torch.float32, device=dev), torch.empty_like(q))
        prepared.append((w, hc, q, k, v, ref, got))
    torch.cuda.synchronize()
    free_before = None
    for i, (w, hc, q, k, v, ref, got) in enumerate(prepared):
        print(f"\n  call {i}: S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} head_chunk={hc}", flush=True)
        if i == 1:
            free_before = torch.cuda.mem_get_info(dev)[0]
        out, lse, out_lo = got
        up.upipe_attn_fwd_noalloc(q, k, v, out, out_lo, lse, hc, True)
        torch.cuda.synchronize()
        if i == 1:
            assert torch.cuda.mem_get_info(dev)[0] == free_before, "the second call allocated device memory"
        for name, a, b in (("out", out, ref[0]), ("lse", lse, ref[1]), ("out_lo", out_lo, ref[2])):
            assert bit_equal(a, b), f"call {i}: {name} differs from the workspace forward"
        ro, rl = attention_forward(f64(q), f64(k), f64(v))
        assert_close("out", f64(out), ro, w.dtype, per_item=True)
        assert_close("lse", f64(lse), rl, w.dtype)


def test_noalloc_forward_rejects_a_pool_beyond_the_scratch_array():
    """Host-side check before anything is enqueued (no device memory touched)."""
    S = 70000  # bf16, d = 128, Hkv = head_chunk = 1: about 1 KiB of pool per token
    assert up.upipe_attn_fwd_workspace_bytes(S, 4, 1, 128, 1, 0) > up.NOALLOC_SCRATCH_BYTES
    fake = 0x10000
    rc = up._lib.lib().upipe_attn_fwd_noalloc(fake, fake, fake, fake, None, fake, S, 4, 1, 128, 1, 1, 0, None)
    assert rc == -3 and "static scratch" in up.upipe_last_error()
    assert up.upipe_attn_fwd_workspace_bytes(65000, 4, 1, 128, 1, 0) <= up.NOALLOC_SCRATCH_BYTES
