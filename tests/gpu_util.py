"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle under the stated tolerances."""

import os
import time

import numpy as np
import torch

import long_context_attention_upipe_amd as up

# max |err| <= 2e-2 and ||err||_F / ||ref||_F <= 5e-3 for bf16 inputs;
# <= 1e-4 relative Frobenius for fp32 inputs.
TOL = {"bf16": (2e-2, 5e-3), "fp32": (2e-2, 1e-4)}


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run(q, k, v, do, head_chunk, causal=True, ws=None, doc_offsets=None):
    """Forward then backward on the current device; returns device tensors.
    ``doc_offsets`` (int32 device tensor) selects the packed-document calls."""
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    if ws is None:
        ws = up.workspace(S, Hq, Hkv, d, head_chunk, q.dtype, q.device, "both")
    out, lse, out_lo = up.attention_forward(q, k, v, head_chunk=head_chunk, causal=causal, ws=ws,
                                            doc_offsets=doc_offsets)
    res = {"out": out, "lse": lse}
    if do is not None:
        dq, dk, dv = up.attention_backward(q, k, v, out, do, lse, out_lo, head_chunk=head_chunk, causal=causal, ws=ws,
                                           doc_offsets=doc_offsets)
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


def oracle_parallel(fn, parts, label):
    """[fn(p) for p in parts], evaluated on a thread pool with single-threaded
    BLAS: the oracle's per-row work is numpy elementwise passes, which release
    the GIL but run on one core each. Prints a progress line as parts finish."""
    from concurrent.futures import ThreadPoolExecutor, as_completed

    from threadpoolctl import threadpool_limits

    workers = max(1, min(16, os.cpu_count() or 1, len(parts)))
    results = [None] * len(parts)
    t0 = last = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        futures = {ex.submit(fn, p): i for i, p in enumerate(parts)}
        for n_done, fut in enumerate(as_completed(futures), 1):
            results[futures[fut]] = fut.result()
            now = time.perf_counter()
            if now - last > 20 or n_done == len(parts):
                print(f"   oracle {label}: {n_done}/{len(parts)} parts, {now - t0:.0f}s", flush=True)
                last = now
    return results


def interleaved_parts(n, n_parts):
    """Split range(n) into n_parts strided index sets of near-equal cost when
    the items are sorted by cost."""
    return [np.arange(i, n, n_parts) for i in range(min(n, n_parts))]


def sum64(t, dims, chunk_elems=1 << 24):
    """Sum of a device tensor over ``dims`` (dim 0 included) in float64,
    chunked along dim 0 so no full-size float64 copy is made."""
    acc = None
    chunk = max(1, chunk_elems // max(1, t[0].numel()))
    for s0 in range(0, t.shape[0], chunk):
        part = t[s0:s0 + chunk].double().sum(dim=dims)
        acc = part if acc is None else acc + part
    return acc.cpu().numpy()
