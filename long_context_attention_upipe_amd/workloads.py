"""Seeded synthetic workloads: shapes, seeds and input generators.

This module holds no attention arithmetic. It only draws the inputs (q, k, v,
dO) from seeded normal distributions and picks sample indices, so that the
HIP path and the CPU oracle can be fed the very same values.

Shapes follow the per-GPU Ulysses share of a Llama-3-8B-like model (32 query
heads and 8 kv heads split over 8 GPUs gives 4 query heads and 1 kv head per
GPU) and of a 32B-shaped model (8 query heads, 1 kv head per GPU), at the
sequence lengths the talk reaches (3M tokens with the technique stack, 5M
with UPipe) ["Road to 5 Million Tokens" talk summary, Summary and Chapters;
MaxText long-context article, strategy table: one kv head per chip at most].
The head dim (128) is not fixed by the pages; 128 is the Llama-3 value.

Packed documents (MaxText long-context article: several samples packed into
one long sequence) come as offsets 0 = o_0 <= ... <= o_n = S. The pages give
no length distribution; the workloads here draw document lengths
log-uniformly between a minimum and a maximum (every scale equally likely),
seeded, and cut the last document at S.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem for a single GPU's share of heads."""

    name: str
    S: int
    Hq: int
    Hkv: int
    d: int
    dtype: str  # "bf16" or "fp32"
    head_chunks: tuple
    dout_scaled: bool  # dO ~ N(0,1)/sqrt(S) instead of N(0,1)
    seed: int
    causal: bool = True
    doc_lengths: tuple = ()  # (min, max) of log-uniform document lengths; () = one sequence

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS = {
    "mha_s1k_fp32": Workload("mha_s1k_fp32", 1024, 4, 4, 64, "fp32", (1, 4), False, 1000),
    "llama8b_share_s128k": Workload("llama8b_share_s128k", 131072, 4, 1, 128, "bf16", (1, 2, 4), True, 2000),
    "llama8b_share_s1m": Workload("llama8b_share_s1m", 1048576, 4, 1, 128, "bf16", (1, 2, 4), True, 3000),
    "llama8b_share_s3m": Workload("llama8b_share_s3m", 3145728, 4, 1, 128, "bf16", (1, 2, 4), True, 4000),
    "share32b_s5m": Workload("share32b_s5m", 5242880, 8, 1, 128, "bf16", (1, 2, 4, 8), True, 5000),
    "llama8b_share_s1m_docs": Workload("llama8b_share_s1m_docs", 1048576, 4, 1, 128, "bf16", (1, 2, 4), True, 6000,
                                       doc_lengths=(1024, 262144)),
}


def custom(S, Hq, Hkv, d, dtype="bf16", seed=7, dout_scaled=False, causal=True, name=None):
    """A workload of arbitrary shape (used by parity tests at small sizes)."""
    return Workload(name or f"S{S}_Hq{Hq}_Hkv{Hkv}_d{d}_{dtype}", S, Hq, Hkv, d, dtype,
                    (1,), dout_scaled, seed, causal)


def loguniform_doc_offsets(S: int, min_len: int, max_len: int, seed: int) -> np.ndarray:
    """Offsets (int32, 0 .. S) of documents whose lengths are drawn seeded and
    log-uniformly in [min_len, max_len]; the last document is cut at S."""
    rng = np.random.default_rng(seed)
    offs = [0]
    while offs[-1] < S:
        n = int(round(math.exp(rng.uniform(math.log(min_len), math.log(max_len)))))
        offs.append(min(S, offs[-1] + max(1, n)))
    return np.asarray(offs, dtype=np.int32)


def doc_offsets(w: Workload):
    """The workload's document offsets (int32 numpy), or None for one sequence."""
    if not w.doc_lengths:
        return None
    return loguniform_doc_offsets(w.S, w.doc_lengths[0], w.doc_lengths[1], w.seed + 9)


def doc_boundary_rows(offsets, n_docs: int, seed: int) -> np.ndarray:
    """Seeded sample of positions at document edges: the first two and last
    two positions of up to ``n_docs`` documents."""
    rng = np.random.default_rng(seed)
    offs = np.asarray(offsets, dtype=np.int64)
    nonempty = [m for m in range(len(offs) - 1) if offs[m + 1] > offs[m]]
    pick = rng.choice(nonempty, size=min(n_docs, len(nonempty)), replace=False)
    rows = set()
    for m in pick:
        a, b = int(offs[m]), int(offs[m + 1])
        rows.update(r for r in (a, a + 1, b - 2, b - 1) if a <= r < b)
    return np.array(sorted(rows), dtype=np.int64)


def _normal(shape, seed, device, dtype, slab_dim=None):
    """N(0,1) fp32 draws from a seeded generator, rounded to ``dtype``.

    Large tensors are drawn slab by slab along ``slab_dim`` so that the fp32
    temporary stays small; the values depend only on (shape, seed, device).
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    if slab_dim is None:
        out.copy_(torch.randn(shape, generator=gen, device=device, dtype=torch.float32))
        return out
    for i in range(shape[slab_dim]):
        sl = [slice(None)] * len(shape)
        sl[slab_dim] = i
        sub = list(shape)
        del sub[slab_dim]
        out[tuple(sl)].copy_(torch.randn(sub, generator=gen, device=device, dtype=torch.float32))
    return out


def make_inputs(w: Workload, device="cpu", need_dout=True):
    """Draw q, k, v (and dO) for workload ``w`` on ``device``.

    Seeds: q = seed, k = seed+1, v = seed+2, dO = seed+3. The rounded values
    are the inputs; the oracle reads them back exactly (upcast to fp64).
    """
    dt = w.torch_dtype
    big = w.S * max(w.Hq, w.Hkv) * w.d > (1 << 26)
    slab = 1 if big else None
    q = _normal((w.S, w.Hq, w.d), w.seed, device, dt, slab)
    k = _normal((w.S, w.Hkv, w.d), w.seed + 1, device, dt, slab)
    v = _normal((w.S, w.Hkv, w.d), w.seed + 2, device, dt, slab)
    if not need_dout:
        return q, k, v, None
    dout = _normal((w.S, w.Hq, w.d), w.seed + 3, device, dt, slab)
    if w.dout_scaled:
        # dO ~ N(0,1)/sqrt(S): a loss averaged over S positions
        dout.mul_(1.0 / math.sqrt(w.S))
    return q, k, v, dout


def sample_rows(S: int, n: int, seed: int, tile: int = 128) -> np.ndarray:
    """Seeded sample of row indices: the first and last rows, rows on both
    sides of tile boundaries, and the rest uniform. Sorted, unique."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, S - 1}
    n_tiles = max(1, (S + tile - 1) // tile)
    for t in rng.choice(n_tiles, size=min(n_tiles, max(1, n // 8)), replace=False):
        for r in (int(t) * tile - 1, int(t) * tile, int(t) * tile + tile - 1):
            if 0 <= r < S:
                fixed.add(r)
    fixed = sorted(fixed)[: n]
    rest = n - len(fixed)
    pool = np.setdiff1d(np.arange(S), np.asarray(fixed)) if S <= (1 << 22) else None
    if rest > 0:
        if pool is not None:
            extra = rng.choice(pool, size=min(rest, len(pool)), replace=False)
        else:
            extra = rng.integers(0, S, size=rest)
        fixed = np.union1d(np.asarray(fixed, dtype=np.int64), extra.astype(np.int64))
    return np.unique(np.asarray(fixed, dtype=np.int64))


def tail_keys(S: int, n: int, window: int, seed: int) -> np.ndarray:
    """Seeded sample of key indices in the last ``window`` positions (always
    including the last key and the start of the window)."""
    rng = np.random.default_rng(seed)
    lo = max(0, S - window)
    keys = {S - 1, lo}
    span = S - lo
    if span > 2:
        keys.update(int(x) for x in rng.choice(np.arange(lo, S), size=min(n, span), replace=False))
    return np.array(sorted(keys), dtype=np.int64)


def make_block_inputs(S: int, Dm: int, Hq: int, Hkv: int, d: int, seed: int, device="cpu"):
    """Inputs of the attention block: x [S, Dm] ~ N(0,1) and torch-Linear
    weights wq [Hq*d, Dm], wk, wv [Hkv*d, Dm] ~ N(0, 1/Dm), wo [Dm, Hq*d] ~
    N(0, 1/(Hq*d)) (unit-variance projections), all rounded to bf16.
    Seeds: x = seed, wq = seed+1, wk = seed+2, wv = seed+3, wo = seed+4."""
    dt = torch.bfloat16
    x = _normal((S, Dm), seed, device, dt)
    wq = _normal((Hq * d, Dm), seed + 1, device, torch.float32).mul_(1 / math.sqrt(Dm)).to(dt)
    wk = _normal((Hkv * d, Dm), seed + 2, device, torch.float32).mul_(1 / math.sqrt(Dm)).to(dt)
    wv = _normal((Hkv * d, Dm), seed + 3, device, torch.float32).mul_(1 / math.sqrt(Dm)).to(dt)
    wo = _normal((Dm, Hq * d), seed + 4, device, torch.float32).mul_(1 / math.sqrt(Hq * d)).to(dt)
    return x, wq, wk, wv, wo
