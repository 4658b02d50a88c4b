"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle under the stated tolerances."""

import os
import time

import sys

import numpy as np
import torch

import long_context_attention_upipe_amd as up

# max |err| <= 2e-2 and ||err||_F / ||ref||_F <= 5e-3 for bf16 inputs;
# <= 1e-4 relative Frobenius for fp32 inputs.
TOL = {"bf16": (2e-2, 5e-3), "fp32": (2e-2, 1e-4)}


def grad_scale(w):
    """Factor that brings gradients back to unit dO scale: sqrt(S) for the
    workloads whose dO is drawn as N(0,1)/sqrt(S), else 1."""
    import math

    return math.sqrt(w.S) if w.dout_scaled else 1.0


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


def assert_close(name, got, ref, dtype, rel_only=False, grad_scale=1.0, per_item=False, elem_floor=1.0):
    """max |err| and relative Frobenius error of a tensor against the oracle.

    grad_scale: gradients are linear in dO, so for workloads whose dO is drawn
    at a reduced scale (N(0,1)/sqrt(S)) both sides are multiplied back to unit
    dO scale (grad_scale = sqrt(S)) before the max-abs bound is applied, as
    |err| <= 2e-2 * max(|ref|, 1) per element.
    per_item: also bound the error of every item along axis 0 (a sampled row
    or key): ||err_i|| <= PER_ITEM_FACTOR * rel_tol * max(||ref_i||, rms_i
    ||ref_i||), so one wrong row or key fails even when the tensor-wide norm
    would absorb it."""
    max_abs_tol, rel_tol = TOL[dtype]
    if rel_only:
        max_abs_tol = float("inf")
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    max_abs, rel = errors(got * grad_scale, ref * grad_scale)
    msg = f"    {name:4s} max_abs={max_abs:.3e}" + (f" (x{grad_scale:.4g}, unit dO)" if grad_scale != 1.0 else "") \
        + f" rel_fro={rel:.3e}"
    if grad_scale != 1.0 or elem_floor != 1.0:
        # At unit dO scale gradient entries reach ~10 (a key's dV sums dO over
        # the rows that see it), where bf16's own half-ulp, 2^-8 |x|, exceeds
        # 2e-2: the bound is absolute for |ref| <= floor and relative above.
        # floor = 1, or (elem_floor="rms") the tensor's RMS at unit scale, for
        # weight gradients summed over every token, whose rounding error grows
        # with the size of the summed terms rather than with the sum.
        # elem_floor="row": each item's (axis-0 row's) own RMS, for a gradient
        # whose rows differ in scale by orders of magnitude (a vocabulary's
        # rows: the labelled ones carry the one-hot term, the rest only
        # softmax mass).
        g, r_ = got * grad_scale, ref * grad_scale
        if elem_floor == "rms":
            # an all-zero reference (e.g. dq of a one-token sequence, where
            # the only key takes softmax weight 1) keeps the absolute floor 1
            floor = float(np.sqrt(np.mean(r_ ** 2))) or 1.0
        elif elem_floor == "row":
            n = r_.shape[0]
            floor = np.sqrt(np.mean(r_.reshape(n, -1) ** 2, axis=1)).reshape((n,) + (1,) * (r_.ndim - 1))
            floor = np.maximum(floor, 1e-30)
        else:
            floor = float(elem_floor)
        max_abs = float((np.abs(g - r_) / np.maximum(np.abs(r_), floor)).max()) if ref.size else 0.0
        msg += f" max_err/max(|ref|,{elem_floor})={max_abs:.3e}"
    worst = None
    if per_item and ref.shape[0] > 1:
        n = ref.shape[0]
        err_i = np.linalg.norm((got - ref).reshape(n, -1), axis=1)
        ref_i = np.linalg.norm(ref.reshape(n, -1), axis=1)
        floor = float(np.sqrt(np.mean(ref_i ** 2)))
        ratio = err_i / np.maximum(ref_i, floor) if floor > 0 else err_i
        worst = (float(ratio.max()), int(ratio.argmax()))
        msg += f" worst_item={worst[0]:.3e}@{worst[1]}"
    print(msg, flush=True)
    assert max_abs <= max_abs_tol and rel <= rel_tol, \
        f"{name}: max_abs={max_abs:.3e} (tol {max_abs_tol}) rel_fro={rel:.3e} (tol {rel_tol})"
    if worst is not None:
        assert worst[0] <= PER_ITEM_FACTOR * rel_tol, \
            f"{name}: item {worst[1]} off by {worst[0]:.3e} of its norm (tol {PER_ITEM_FACTOR * rel_tol})"


# One item (row or key) may be worse than the tensor as a whole, which averages
# many items; 4x the tensor-wide relative bound still fails any item whose
# value is wrong rather than rounded.
PER_ITEM_FACTOR = 4.0


PYTEST_CONFIG = None  # set by conftest.pytest_configure


def progress(msg):
    """Print a progress line straight to the terminal, past pytest's output
    capture, so that a minutes-long GPU case run under -q shows it is
    advancing (its kernels finishing) while it runs."""
    capman = PYTEST_CONFIG.pluginmanager.getplugin("capturemanager") if PYTEST_CONFIG else None
    if capman is None:
        print(msg, flush=True)
        return
    with capman.global_and_fixture_disabled():
        sys.stdout.write(msg + "\n")
        sys.stdout.flush()


def bit_equal(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                       b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))


class OracleJobs:
    """Oracle work on a host thread pool that runs while the GPU computes.

    Every BLAS call is held to ONE thread while the pool runs: OpenBLAS
    (pthreads build) called concurrently from several threads, each running
    its own multi-threaded GEMMs, returned wrong products on a 16-core EPYC
    host (a full-tensor oracle run per head in 4 threads x 4 BLAS threads
    differed from the per-row oracle on 13,196 of 131,072 rows, on different
    rows from run to run), while single-threaded calls from many threads gave
    the same numbers as sequential runs. Parallelism comes from splitting the
    work into parts instead (the per-row work is numpy elementwise passes
    plus matrix products, which release the GIL). map() submits and returns
    at once; gather() blocks, printing a progress line as parts finish."""

    def __init__(self, workers=None):
        from concurrent.futures import ThreadPoolExecutor

        from threadpoolctl import threadpool_limits

        cores = max(1, min(16, os.cpu_count() or 1))
        self.workers = workers or max(1, cores - 1)  # one core left for the GPU's host thread
        self._limits = threadpool_limits(1)
        self._ex = ThreadPoolExecutor(self.workers)
        self._t0 = time.perf_counter()

    def map(self, fn, parts, label):
        return label, [self._ex.submit(fn, p) for p in parts]

    def gather(self, job):
        from concurrent.futures import as_completed

        label, futures = job
        last = time.perf_counter()
        for n_done, fut in enumerate(as_completed(futures), 1):
            fut.result()
            now = time.perf_counter()
            if now - last > 20 or n_done == len(futures):
                progress(f"   oracle {label}: {n_done}/{len(futures)} parts, {now - self._t0:.0f}s")
                last = now
        return [f.result() for f in futures]

    def close(self):
        self._ex.shutdown(wait=True, cancel_futures=True)
        self._limits.restore_original_limits()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


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
