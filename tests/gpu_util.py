"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle under the stated tolerances."""

import numpy as np
import torch

import long_context_attention_upipe_amd as up

# max |err| <= 2e-2 and ||err||_F / ||ref||_F <= 5e-3 for bf16 inputs;
# <= 1e-4 relative Frobenius for fp32 inputs.
TOL = {"bf16": (2e-2, 5e-3), "fp32": (2e-2, 1e-4)}


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run(q, k, v, do, head_chunk, causal=True, ws=None):
    """Forward then backward on the current device; returns device tensors."""
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    if ws is None:
        ws = up.workspace(S, Hq, Hkv, d, head_chunk, q.dtype, q.device, "both")
    out, lse, out_lo = up.attention_forward(q, k, v, head_chunk=head_chunk, causal=causal, ws=ws)
    res = {"out": out, "lse": lse}
    if do is not None:
        dq, dk, dv = up.attention_backward(q, k, v, out, do, lse, out_lo, head_chunk=head_chunk, causal=causal, ws=ws)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return res


def errors(got, ref):
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm(diff.ravel()) / denom) if denom > 0 else float(np.linalg.norm(diff.ravel()))
    return max_abs, rel


def assert_close(name, got, ref, dtype, rel_only=False):
    max_abs_tol, rel_tol = TOL[dtype]
    if rel_only:
        max_abs_tol = float("inf")
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    max_abs, rel = errors(got, ref)
    print(f"    {name:4s} max_abs={max_abs:.3e} rel_fro={rel:.3e}", flush=True)
    assert max_abs <= max_abs_tol and rel <= rel_tol, \
        f"{name}: max_abs={max_abs:.3e} (tol {max_abs_tol}) rel_fro={rel:.3e} (tol {rel_tol})"


def bit_equal(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                       b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))
