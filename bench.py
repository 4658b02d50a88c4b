#!/usr/bin/env python3
"""Benchmark: causal GQA attention forward+backward, UPipe head chunks, one GPU.

One step = upipe_attn_fwd + upipe_attn_bwd over the whole workload: the
chunk planner, the pack copies (the stand-in for the Ulysses exchange), the
forward kernel, the unpack, the D pre-pass, the dK/dV and dQ kernels and the
final copies, every head chunk reusing one fixed pool. Inputs are resident in
HBM before the timed region starts.

Prints ONE JSON line. `value` is algorithmic attention TFLOP/s for fwd+bwd:
F = 14 * d * Hq * S(S+1)/2 per step (fwd 4*d per unmasked (row, key) pair:
Q K^T and P V; bwd 10*d: the Q K^T recompute, dP, dV, dK and dQ). Masked
pairs, softmax work and any extra recompute are not counted.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--head-chunk HC] [--no-sweep] [--no-residual-run] [--no-cpu-baseline]

After the timed headline run, every other head_chunk of the workload runs
(1 warmup + 2 steps each by default) so the line carries the chunk-size
trade-off: TFLOP/s and peak HBM per head_chunk (`head_chunk_sweep`). One more
step at the headline head_chunk runs without out_lo (the forward's stored
rounding residual of out) to report peak HBM when D comes from out alone.
Then one call of the fused deterministic backward (upipe_attn_bwd_fused) on
the same workload (`fused_backward`: time, TFLOP/s, its speed against the
two-kernel backward timed above, pool and peak HBM), and the attention block,
loss and MLP legs (`block_fwd`, `tiled_loss`, `tiled_mlp`).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s & % bf16 MFMA peak at 1M-5M tokens; peak HBM"
# MI355X dense bf16 MFMA peak: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz.
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_MFMA_TFLOPS = 157.3
GIB = float(1 << 30)

# Algorithmic FLOPs per unmasked (row, key) pair and head, per kernel, in units
# of d: fwd = Q K^T + P V; dK/dV kernel = Q K^T (recompute) + dP + dV + dK;
# dQ kernel = dQ only (its Q K^T and dP recomputes duplicate the dK/dV kernel's).
ALGO_FLOPS_PER_PAIR_D = {"attn_fwd": 4, "attn_bwd_dkdv": 8, "attn_bwd_dq": 2}
EXEC_FLOPS_PER_PAIR_D = {"attn_fwd": 4, "attn_bwd_dkdv": 8, "attn_bwd_dq": 6}


# The device code of the three attention kernels is defined by these headers
# alone (tiles, grid mapping, arithmetic); HBM counters taken on other sources
# do not describe them.
ATTN_KERNEL_SOURCES = ("attn_bf16.hpp", "attn_fwd.hpp", "attn_bwd.hpp", "common.hpp", "lds_tiles.hpp")


def kernel_source_hash() -> str:
    """sha256 over the HIP headers that define the attention kernels."""
    import hashlib

    d = os.path.join(ROOT, "long_context_attention_upipe_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(ATTN_KERNEL_SOURCES):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def algo_bytes(kernel: str, w, head_chunk: int) -> int:
    """Algorithmic HBM bytes of one launch: every input read once, every output
    written once, for the head_chunk query heads of a chunk and their kv heads.
    forward: Q, K, V in, O, LSE out; dK/dV and dQ: Q, dO, K, V, LSE, D in and
    their own outputs out."""
    es = 2 if w.dtype == "bf16" else 4
    G = w.Hq // w.Hkv
    nkv = max(1, head_chunk // G)
    U = w.S * w.d * es
    rows = head_chunk * w.S * 4  # one fp32 per (row, head)
    if kernel == "attn_fwd":
        return 2 * head_chunk * U + 2 * nkv * U + rows
    if kernel == "attn_bwd_dkdv":
        return 2 * head_chunk * U + 2 * nkv * U + 2 * rows + 2 * nkv * U
    if kernel == "attn_bwd_dq":
        return 2 * head_chunk * U + 2 * nkv * U + 2 * rows + head_chunk * U
    raise KeyError(kernel)


def measured_traffic(kernel: str, workload: str, head_chunk: int):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE runs recorded in
    profiles/traffic.json, or None if none were taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        entries = json.load(f).get("entries", [])
    src = kernel_source_hash()
    for e in entries:
        if (e["kernel"], e["workload"], e["head_chunk"], e["src_sha256"]) == (kernel, workload, head_chunk, src):
            return int(e["read_bytes_per_launch"] + e["write_bytes_per_launch"])
    return None


def pairs(S: int, causal: bool, offsets=None) -> int:
    """Unmasked (row, key) pairs of one head: the causal triangle, the full
    square, or their sum over packed documents."""
    if offsets is None:
        return S * (S + 1) // 2 if causal else S * S
    lens = [int(b) - int(a) for a, b in zip(offsets[:-1], offsets[1:])]
    return sum(n * (n + 1) // 2 if causal else n * n for n in lens)


def prefix_offsets(offsets, n: int):
    """Document offsets of the first n positions (None stays None)."""
    if offsets is None:
        return None
    cut = [int(o) for o in offsets if int(o) < n]
    return cut + [n]


def cpu_baseline(w, q, k, v, do, s_prefix: int):
    """Time the fp64 CPU oracle (as it stands) on the first s_prefix positions
    of the same inputs: a causal fwd+bwd of that prefix, all heads."""
    import numpy as np

    from oracle.attention import attention_backward  # checker only: the CPU leg

    try:
        import threadpoolctl

        threads = max(int(i.get("num_threads", 1)) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    from long_context_attention_upipe_amd.workloads import doc_offsets

    sl = slice(0, s_prefix)
    arrs = [t[sl].float().cpu().numpy().astype(np.float64) for t in (q, k, v, do)]
    offs = prefix_offsets(doc_offsets(w), s_prefix)
    t0 = time.perf_counter()
    attention_backward(*arrs, causal=w.causal, doc_offsets=offs)  # recomputes the forward inside
    dt = time.perf_counter() - t0
    flops = 14 * w.d * w.Hq * pairs(s_prefix, w.causal, offs)
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
    except OSError:
        pass
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "cpu_model": cpu_model,
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle, causal fwd+bwd of the first {s_prefix} positions of the same "
                  f"inputs (Hq={w.Hq}, Hkv={w.Hkv}, d={w.d}"
                  + (f", {len(offs) - 1} documents" if offs is not None else "") + f"), {dt:.1f} s",
        "seconds": round(dt, 3),
    }


def run_one(w, head_chunk: int, steps: int, warmup: int, dev, residual: bool = True):
    import torch

    import long_context_attention_upipe_amd as up
    from long_context_attention_upipe_amd.workloads import doc_offsets, make_inputs

    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    q, k, v, do = make_inputs(w, device=dev)
    out = torch.empty_like(q)
    # out's rounding residual, for D (residual=False: D from out alone)
    out_lo = torch.empty_like(q) if (residual and q.dtype == torch.bfloat16) else None
    lse = torch.empty((w.Hq, w.S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    code = up.dtype_code(q.dtype)
    ws_bytes = max(up.upipe_attn_fwd_workspace_bytes(w.S, w.Hq, w.Hkv, w.d, head_chunk, code),
                   up.upipe_attn_bwd_workspace_bytes(w.S, w.Hq, w.Hkv, w.d, head_chunk, code))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    offsets = doc_offsets(w)

    if offsets is None:
        def fwd():
            up.upipe_attn_fwd(q, k, v, out, out_lo, lse, head_chunk, w.causal, ws, stream)

        def bwd():
            up.upipe_attn_bwd(q, k, v, out, out_lo, do, lse, dq, dk, dv, head_chunk, w.causal, ws, stream)
    else:
        offs_t = torch.from_numpy(offsets).to(dev)
        up._lib._require_docs(q, offs_t)  # values checked once, outside the timed region

        def fwd():
            up.upipe_attn_fwd_docs(q, k, v, out, out_lo, lse, head_chunk, w.causal, offs_t, ws, stream,
                                   check_offsets=False)

        def bwd():
            up.upipe_attn_bwd_docs(q, k, v, out, out_lo, do, lse, dq, dk, dv, head_chunk, w.causal, offs_t, ws, stream,
                                   check_offsets=False)

    def wait_reporting(what):
        up.wait_reporting(what, dev, prefix="[bench]")

    for _ in range(warmup):
        up.upipe_profile_reset()
        up.upipe_profile_enable(True)
        fwd()
        bwd()
        wait_reporting("warmup")
        up.upipe_profile_enable(False)
    up.upipe_profile_reset()
    torch.cuda.synchronize(dev)
    print(f"[bench] warmup done: {w.name} head_chunk={head_chunk}", file=sys.stderr, flush=True)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    up.upipe_profile_reset()
    up.upipe_profile_enable(True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    wait_reporting("timed")
    t1 = time.perf_counter()
    up.upipe_profile_enable(False)
    prof = up.upipe_profile_read()
    up.upipe_profile_reset()

    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    ms_per_step = (t1 - t0) * 1000.0 / steps
    P = pairs(w.S, w.causal, offsets)
    f_fwd = 4 * w.d * w.Hq * P
    f_bwd = 10 * w.d * w.Hq * P
    peak_alloc = torch.cuda.max_memory_allocated(dev) - base
    kernels = {}
    for name, (launches, total_ms) in prof.items():
        avg = total_ms / max(1, launches)
        entry = {"launches": launches, "avg_ms": round(avg, 4), "total_ms_per_step": round(total_ms / steps, 3)}
        if name in ALGO_FLOPS_PER_PAIR_D:
            per_launch = ALGO_FLOPS_PER_PAIR_D[name] * w.d * head_chunk * P
            execd = EXEC_FLOPS_PER_PAIR_D[name] * w.d * head_chunk * P
            entry["algo_tflops"] = round(per_launch / (avg / 1e3) / 1e12, 2)
            entry["exec_tflops"] = round(execd / (avg / 1e3) / 1e12, 2)
        kernels[name] = entry
    res = {
        "head_chunk": head_chunk,
        "ms_per_step": ms_per_step,
        "fwd_ms": fwd_ms,
        "bwd_ms": bwd_ms,
        "tflops": (f_fwd + f_bwd) / (ms_per_step / 1e3) / 1e12,
        "fwd_tflops": f_fwd / (fwd_ms / 1e3) / 1e12,
        "bwd_tflops": f_bwd / (bwd_ms / 1e3) / 1e12,
        "peak_hbm_gib": peak_alloc / GIB,
        "out_lo_gib": (out_lo.numel() * out_lo.element_size() / GIB) if out_lo is not None else 0.0,
        "workspace_gib": ws_bytes / GIB,
        "kernels": kernels,
    }
    tensors = (q, k, v, do)
    del out, out_lo, lse, dq, dk, dv, ws
    return res, tensors


def block_sweep(w, dev, chunks, warmup=1):
    """The attention block forward (q, k, v projections of each head chunk,
    attention, its share of the output projection) at every head_chunk: time
    for one call, peak HBM over the call (x, weights, y, lse and the pool; no
    q, k, v or o of all heads exists) and the pool. Dm = Hq * d (the share's
    heads as the whole model)."""
    import torch

    import long_context_attention_upipe_amd as up
    from long_context_attention_upipe_amd.workloads import make_block_inputs

    Dm = w.Hq * w.d
    rows = []
    for hc in chunks:
        torch.cuda.synchronize(dev)
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        x, wq, wk, wv, wo = make_block_inputs(w.S, Dm, w.Hq, w.Hkv, w.d, seed=w.seed + 50, device=dev)
        y = torch.empty((w.S, Dm), dtype=torch.float32, device=dev)
        lse = torch.empty((w.Hq, w.S), dtype=torch.float32, device=dev)
        ws = torch.empty(up.upipe_attn_block_fwd_workspace_bytes(w.S, Dm, w.Hq, w.Hkv, w.d, hc), dtype=torch.uint8,
                         device=dev)
        for _ in range(warmup):
            up.upipe_attn_block_fwd(x, wq, wk, wv, wo, y, None, lse, w.Hq, w.Hkv, hc, True, ws)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        up.upipe_attn_block_fwd(x, wq, wk, wv, wo, y, None, lse, w.Hq, w.Hkv, hc, True, ws)
        torch.cuda.synchronize(dev)
        ms = (time.perf_counter() - t0) * 1e3
        attn = 4 * w.d * w.Hq * pairs(w.S, True)
        proj = 2 * w.S * Dm * (w.Hq + 2 * w.Hkv) * w.d + 2 * w.S * w.Hq * w.d * Dm
        rows.append({"head_chunk": hc, "ms": round(ms, 2), "tflops": round((attn + proj) / (ms / 1e3) / 1e12, 2),
                     "peak_hbm_gib": round((torch.cuda.max_memory_allocated(dev) - base) / GIB, 4),
                     "pool_gib": round(ws.numel() / GIB, 4)})
        print(f"[bench] block fwd head_chunk={hc}: {ms:.1f} ms, peak {rows[-1]['peak_hbm_gib']:.2f} GiB",
              file=sys.stderr, flush=True)
        del y, lse, ws
        # backward with o recomputed: x, weights, dy, the fp32 gradients and
        # the pool; one timed call (its kernels are warm from the forward)
        torch.cuda.synchronize(dev)
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev) - sum(t.numel() * t.element_size() for t in (x, wq, wk, wv, wo))
        dy = torch.randn((w.S, Dm), generator=torch.Generator(device=dev).manual_seed(w.seed + 56), device=dev,
                         dtype=torch.float32).to(torch.bfloat16)
        grads = [torch.empty(t.shape, dtype=torch.float32, device=dev) for t in (x, wq, wk, wv, wo)]
        ws = torch.empty(up.upipe_attn_block_bwd_workspace_bytes(w.S, Dm, w.Hq, w.Hkv, w.d, hc, True),
                         dtype=torch.uint8, device=dev)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        up.upipe_attn_block_bwd(x, wq, wk, wv, wo, dy, None, None, *grads, w.Hq, w.Hkv, hc, True, ws)
        torch.cuda.synchronize(dev)
        ms_b = (time.perf_counter() - t0) * 1e3
        attn_b = 14 * w.d * w.Hq * pairs(w.S, True)  # forward again (4d) + backward (10d)
        proj_b = 2 * w.S * Dm * w.d * (3 * (w.Hq + 2 * w.Hkv) + 2 * w.Hq)
        rows[-1].update({"bwd_ms": round(ms_b, 2), "bwd_tflops": round((attn_b + proj_b) / (ms_b / 1e3) / 1e12, 2),
                         "bwd_peak_hbm_gib": round((torch.cuda.max_memory_allocated(dev) - base) / GIB, 4),
                         "bwd_pool_gib": round(ws.numel() / GIB, 4)})
        print(f"[bench] block bwd head_chunk={hc}: {ms_b:.1f} ms, peak {rows[-1]['bwd_peak_hbm_gib']:.2f} GiB",
              file=sys.stderr, flush=True)
        del x, wq, wk, wv, wo, dy, grads, ws
    return {"Dm": Dm, "flops": "attention 4*d*Hq*S(S+1)/2 + projections 2*S*Dm*(Hq+2*Hkv)*d + 2*S*Hq*d*Dm",
            "bwd": "o recomputed; attention 14*d*Hq*S(S+1)/2 (forward again + backward) + projections "
                   "2*S*Dm*d*(3*(Hq+2*Hkv) + 2*Hq) (q, k, v again; dO; dWq, dWk, dWv; dx; dWo)",
            "sweep": rows}


def loss_leg(dev, S=131072, Dm=4096, V=128256, tile=4096):
    """The sequence-tiled cross-entropy, forward and backward (loss, dh, dW),
    on S tokens of a Llama-3-sized head (Dm 4096, vocabulary 128,256): one
    timed call after one warm-up, its peak HBM and its bounded buffer against
    the [S, V] fp32 logits it never forms."""
    import torch

    import long_context_attention_upipe_amd as up

    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    h = torch.randn((S, Dm), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn((V, Dm), generator=g, device=dev) / Dm ** 0.5).to(torch.bfloat16)
    labels = torch.randint(0, V, (S,), generator=g, device=dev, dtype=torch.int32)
    loss = torch.empty(S, device=dev)
    dh = torch.empty_like(h)
    dw = torch.empty((V, Dm), device=dev)
    ws = torch.empty(up.upipe_ce_loss_workspace_bytes(S, Dm, V, tile, True), dtype=torch.uint8, device=dev)
    up.upipe_ce_loss_tiled(h, w, labels, loss, dh, dw, tile, 1.0 / S, ws)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    up.upipe_ce_loss_tiled(h, w, labels, loss, dh, dw, tile, 1.0 / S, ws)
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1e3
    flops = 6 * S * Dm * V
    res = {"S": S, "Dm": Dm, "V": V, "tile": tile, "ms": round(ms, 2),
           "tflops": round(flops / (ms / 1e3) / 1e12, 2), "flops": "6*S*Dm*V (logits, dh, dW GEMMs)",
           "peak_hbm_gib": round((torch.cuda.max_memory_allocated(dev) - base) / GIB, 3),
           "buffer_gib": round(ws.numel() / GIB, 3), "full_logits_fp32_gib": round(S * V * 4 / GIB, 2)}
    print(f"[bench] tiled loss: {ms:.1f} ms, {res['tflops']:.1f} TFLOP/s, peak {res['peak_hbm_gib']:.2f} GiB",
          file=sys.stderr, flush=True)
    del h, w, labels, loss, dh, dw, ws
    return res


def mlp_leg(dev, S=131072, Dm=4096, F=14336, tile=4096):
    """The sequence-tiled SwiGLU MLP, forward and backward, on S tokens of a
    Llama-3-8B-sized MLP (Dm 4096, F 14336): one timed fwd+bwd after one
    warm-up, its peak HBM and its bounded buffer against the [S, F] gate, up
    and activation tensors it never forms."""
    import torch

    import long_context_attention_upipe_amd as up

    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(78)
    x = torch.randn((S, Dm), generator=g, device=dev).to(torch.bfloat16)
    wg = (torch.randn((F, Dm), generator=g, device=dev) / Dm ** 0.5).to(torch.bfloat16)
    wu = (torch.randn((F, Dm), generator=g, device=dev) / Dm ** 0.5).to(torch.bfloat16)
    wd = (torch.randn((Dm, F), generator=g, device=dev) / F ** 0.5).to(torch.bfloat16)
    dy = (torch.randn((S, Dm), generator=g, device=dev) / S).to(torch.bfloat16)
    y = torch.empty_like(x)
    dx = torch.empty((S, Dm), device=dev)
    dwg, dwu = torch.empty((F, Dm), device=dev), torch.empty((F, Dm), device=dev)
    dwd = torch.empty((Dm, F), device=dev)
    ws = torch.empty(up.upipe_mlp_workspace_bytes(S, Dm, F, tile, True), dtype=torch.uint8, device=dev)

    def step():
        up.upipe_mlp_tiled_fwd(x, wg, wu, wd, y, tile, ws)
        up.upipe_mlp_tiled_bwd(x, wg, wu, wd, dy, dx, dwg, dwu, dwd, tile, ws)

    step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize(dev)
    ms = (time.perf_counter() - t0) * 1e3
    flops = 11 * 2 * S * Dm * F  # fwd 3 GEMMs; bwd 2 recomputed, da, dx (2), dWg, dWu, dWd
    res = {"S": S, "Dm": Dm, "F": F, "tile": tile, "ms": round(ms, 2),
           "tflops": round(flops / (ms / 1e3) / 1e12, 2), "flops": "11 GEMMs of 2*S*Dm*F (fwd 3, bwd 8 incl. the recomputed gate/up)",
           "peak_hbm_gib": round((torch.cuda.max_memory_allocated(dev) - base) / GIB, 3),
           "buffer_gib": round(ws.numel() / GIB, 3), "untiled_intermediates_bf16_gib": round(3 * S * F * 2 / GIB, 2)}
    print(f"[bench] tiled MLP: {ms:.1f} ms, {res['tflops']:.1f} TFLOP/s, peak {res['peak_hbm_gib']:.2f} GiB",
          file=sys.stderr, flush=True)
    del x, wg, wu, wd, dy, y, dx, dwg, dwu, dwd, ws
    return res


def fused_leg(w, hc, dev, two_kernel_bwd_ms):
    """The fused deterministic backward (upipe_attn_bwd_fused) on the headline
    workload: the same inputs, forward and head_chunk, one timed backward call
    (HIP events on the launch stream), its kernels' averages, pool and peak HBM."""
    import torch

    import long_context_attention_upipe_amd as up
    from long_context_attention_upipe_amd.workloads import make_inputs

    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    q, k, v, do = make_inputs(w, device=dev)
    out, lse, out_lo = up.attention_forward(q, k, v, head_chunk=hc, causal=w.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = up.upipe_attn_bwd_fused_workspace_bytes(w.S, w.Hq, w.Hkv, w.d, hc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    up.upipe_profile_reset()
    up.upipe_profile_enable(True)
    e0.record(stream)
    up.upipe_attn_bwd_fused(q, k, v, out, out_lo, do, lse, dq, dk, dv, hc, w.causal, ws, 0, stream)
    e1.record(stream)
    up.wait_reporting("fused backward", dev, prefix="[bench]")
    up.upipe_profile_enable(False)
    prof = up.upipe_profile_read()
    up.upipe_profile_reset()
    ms = e0.elapsed_time(e1)
    P = pairs(w.S, w.causal)
    kernels = {n: {"launches": c, "avg_ms": round(t / max(1, c), 3)} for n, (c, t) in prof.items()
               if n in ("attn_bwd_fused", "fused_dq_reduce")}
    res = {"head_chunk": hc, "steps": 1, "bwd_ms": round(ms, 2),
           "bwd_tflops": round(10 * w.d * w.Hq * P / (ms / 1e3) / 1e12, 2),
           "two_kernel_bwd_ms": round(two_kernel_bwd_ms, 2),
           "speed_vs_two_kernel": round(two_kernel_bwd_ms / ms, 3),
           "nan_in_dq": bool(torch.isnan(dq.float()).any()),
           "peak_hbm_gib": round((torch.cuda.max_memory_allocated(dev) - base) / GIB, 3),
           "workspace_gib": round(ws_bytes / GIB, 3), "kernels": kernels,
           "flops": "10*d*Hq*pairs (five products per pair, executed once)"}
    print(f"[bench] fused backward: {ms:.1f} ms ({res['bwd_tflops']:.1f} TFLOP/s), two-kernel {two_kernel_bwd_ms:.1f} ms",
          file=sys.stderr, flush=True)
    del q, k, v, do, out, lse, out_lo, dq, dk, dv, ws
    return res


def roofline(w, res, head_chunk):
    """Roofline entry for the attention kernel with the most time per step."""
    attn = {n: e for n, e in res["kernels"].items() if n in ALGO_FLOPS_PER_PAIR_D}
    name = max(attn, key=lambda n: attn[n]["total_ms_per_step"])
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    achieved = attn[name]["algo_tflops"]
    traffic = measured_traffic(name, w.name, head_chunk)
    ab = algo_bytes(name, w, head_chunk)
    return {
        "kernel": name,
        "bound": "mfma",
        "achieved": achieved,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "algo_bytes": ab,
        "traffic_over_algo_bytes": round(traffic / ab, 1) if traffic else None,
        "per_unit": f"{ALGO_FLOPS_PER_PAIR_D[name]}*d FLOP per unmasked (row, key) pair and head; "
                    f"{head_chunk} heads x "
                    + ("S(S+1)/2" if not w.doc_lengths else "the sum over documents of L(L+1)/2")
                    + " pairs per launch",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama8b_share_s1m")
    ap.add_argument("--head-chunk", type=int, default=None, help="default: the workload's smallest")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the head_chunk sweep (by default every other head_chunk of the workload runs after "
                         "the headline, --sweep-warmup/--sweep-steps each, for the peak-HBM curve)")
    ap.add_argument("--sweep-chunks", default=None, help="comma-separated head_chunk values for the sweep")
    ap.add_argument("--sweep-steps", type=int, default=2)
    ap.add_argument("--sweep-warmup", type=int, default=1)
    ap.add_argument("--no-block", action="store_true",
                    help="skip the attention-block forward sweep (projections around the chunk loop)")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused deterministic backward leg")
    ap.add_argument("--no-loss", action="store_true", help="skip the sequence-tiled cross-entropy leg")
    ap.add_argument("--no-mlp", action="store_true", help="skip the sequence-tiled MLP leg")
    ap.add_argument("--no-residual-run", action="store_true",
                    help="skip the one-step run without out_lo (peak HBM when D comes from out alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-prefix", type=int, default=32768, help="positions in the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 launches), to scale HBM counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the path "
              "has no collectives; per-GPU shares are independent under head sharding.", file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_attention_upipe_amd.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (no CPU fallback)", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        a = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "launches": 3}), flush=True)
        return
    w = WORKLOADS[args.workload]
    hc = args.head_chunk or min(w.head_chunks)
    props = torch.cuda.get_device_properties(dev)
    print(f"[bench] {props.name} CUs={props.multi_processor_count} workload={w.name} S={w.S} "
          f"Hq={w.Hq} Hkv={w.Hkv} d={w.d} {w.dtype} head_chunk={hc}", file=sys.stderr, flush=True)

    res, tensors = run_one(w, hc, args.steps, args.warmup, dev)
    print(f"[bench] timed: {res['ms_per_step']:.1f} ms/step, {res['tflops']:.1f} TFLOP/s", file=sys.stderr,
          flush=True)
    del tensors  # every run draws its own inputs (same seeds): keep one set resident at a time
    sweep = []
    if not args.no_sweep:
        chunks = [int(x) for x in args.sweep_chunks.split(",")] if args.sweep_chunks else list(w.head_chunks)
        for h in chunks:
            r = res if h == hc else run_one(w, h, args.sweep_steps, args.sweep_warmup, dev)[0]
            entry = {k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in r.items() if k_ != "kernels"}
            entry["steps"] = args.steps if h == hc else args.sweep_steps
            sweep.append(entry)
            print(f"[bench] sweep head_chunk={h}: {r['tflops']:.1f} TFLOP/s peak {r['peak_hbm_gib']:.2f} GiB",
                  file=sys.stderr, flush=True)
    no_res = None
    if not args.no_residual_run and w.dtype == "bf16":
        r = run_one(w, hc, 1, 0, dev, residual=False)[0]
        no_res = {"head_chunk": hc, "peak_hbm_gib": round(r["peak_hbm_gib"], 4), "tflops": round(r["tflops"], 2),
                  "steps": 1, "warmup": 0}
        print(f"[bench] without out_lo: peak {r['peak_hbm_gib']:.2f} GiB", file=sys.stderr, flush=True)

    fused = None
    if not args.no_fused and w.dtype == "bf16" and w.d == 128 and not w.doc_lengths:
        fused = fused_leg(w, hc, dev, res["bwd_ms"])

    block = None
    if not args.no_block and w.dtype == "bf16" and not w.doc_lengths:
        block = block_sweep(w, dev, list(w.head_chunks))
    loss_res = None if args.no_loss else loss_leg(dev)
    mlp_res = None if args.no_mlp else mlp_leg(dev)

    cpu = None
    if not args.no_cpu_baseline:
        from long_context_attention_upipe_amd.workloads import make_inputs

        # the same seeded inputs, drawn again on the device and cut to the prefix
        q, k, v, do = (t[:min(args.cpu_prefix, w.S)] for t in make_inputs(w, device=dev))
        cpu = cpu_baseline(w, q, k, v, do, min(args.cpu_prefix, w.S))
        del q, k, v, do
        print(f"[bench] cpu oracle: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads", file=sys.stderr,
              flush=True)

    config = {"workload": w.name, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "head_chunk": hc,
              "causal": w.causal, "parallelism": "1 GPU's Ulysses head share, UPipe head chunks"}
    if w.doc_lengths:
        from long_context_attention_upipe_amd.workloads import doc_offsets

        config["documents"] = len(doc_offsets(w)) - 1
        config["doc_lengths_loguniform"] = list(w.doc_lengths)
    line = {
        "metric": METRIC,
        "value": round(res["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, dO ~ N(0,1)/sqrt(S), drawn on device)",
        "config": config,
        "pct_bf16_peak": round(100.0 * res["tflops"] / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(res["fwd_ms"], 3),
        "bwd_ms": round(res["bwd_ms"], 3),
        "fwd_tflops": round(res["fwd_tflops"], 2),
        "bwd_tflops": round(res["bwd_tflops"], 2),
        "peak_hbm_gib": round(res["peak_hbm_gib"], 3),
        "out_lo_gib": round(res["out_lo_gib"], 3),
        "peak_hbm_without_out_lo": no_res,
        "workspace_gib": round(res["workspace_gib"], 3),
        "roofline": roofline(w, res, hc),
        "cpu_baseline": cpu,
        "kernels": res["kernels"],
    }
    if sweep:
        line["head_chunk_sweep"] = sweep
    if fused:
        line["fused_backward"] = fused
    if block:
        line["block_fwd"] = block
    if loss_res:
        line["tiled_loss"] = loss_res
    if mlp_res:
        line["tiled_mlp"] = mlp_res
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
