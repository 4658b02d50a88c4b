"""Plain fp64 CPU oracle of the attention block around the chunked attention:
the layer's q, k, v projections, causal GQA attention, the output projection.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it, and it shares nothing with the HIP library.

Source: "Road to 5 Million Tokens: Breaking Barriers in Long Context
Training" talk summary, Chapters: in the Q&A the head batching is said to
target the layer's Q, K and V matrices (each one a full-sequence tensor); the
chapter on processing heads in batches runs a group of heads at a time
through buffers the previous group used. Computing a chunk's q, k, v from the
layer input right before its attention, and its share of the output
projection right after, is what keeps those full-sequence tensors for all
heads from existing at once. The block computes, per head h (kv head g):

    q_h = x Wq_h^T,  k_g = x Wk_g^T,  v_g = x Wv_g^T      (torch Linear layout:
                                                         W[out_features, in_features])
    o_h = attention(q_h, k_g, v_g)                       (oracle.attention)
    y   = sum_h o_h Wo_h^T                               (Wo_h: Wo's columns of head h)

Readings where the pages are silent:
  * Linear weights are in torch's [out, in] layout, no biases;
  * head h occupies features h*d .. h*d + d - 1 of q (and of the output
    projection's input), kv head g features g*d .. of k and v;
  * x, the weights, q, k, v and the attention output are bf16 tensors: the
    block's intermediate q, k, v and o are the bf16 values a bf16 layer
    would hand on, i.e. each is the exact product rounded to float32 and then
    to bf16, round to nearest even (``round_bf16``); y is returned in fp64.

The backward (:func:`attention_block_backward`) is the chain rule through the
same steps, for the upstream gradient dy of y:

    do_h   = dy Wo_h                     dWo_h = dy^T o_h
    dq_h, dk_g, dv_g = attention backward (oracle.attention) from do
    dx     = sum_h dq_h Wq_h + sum_g (dk_g Wk_g + dv_g Wv_g)
    dWq_h  = dq_h^T x,  dWk_g = dk_g^T x,  dWv_g = dv_g^T x

Reading for the backward: the forward's bf16 roundings are straight-through
(their derivative is taken as 1) and the gradients themselves are kept exact
in fp64; a bf16 layer would round do, dq, dk and dv once more, which the
comparison's bf16 tolerance covers.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_backward, attention_forward, forward_rows

__all__ = ["round_bf16", "attention_block_forward", "attention_block_rows", "attention_block_backward"]


def round_bf16(x) -> np.ndarray:
    """float64 -> float32 -> bf16 (round to nearest even), returned as float64:
    the value a bf16 tensor holds after an fp32 computation is stored."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x32.view(np.uint32).astype(np.uint64)
    # add half an ulp of bf16 (0x7FFF) plus the lowest kept bit, for ties to even
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16 << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def attention_block_forward(x, wq, wk, wv, wo, n_q_heads: int, n_kv_heads: int, causal: bool = True,
                            round_intermediates: bool = True):
    """y [S, Dm], out [S, Hq, d] and lse [Hq, S] of the attention block on
    x [S, Dm] with wq [Hq*d, Dm], wk, wv [Hkv*d, Dm], wo [Dm, Hq*d]."""
    x, wq, wk, wv, wo = (np.asarray(t, dtype=np.float64) for t in (x, wq, wk, wv, wo))
    S, Dm = x.shape
    d = wq.shape[0] // n_q_heads
    rnd = round_bf16 if round_intermediates else (lambda t: t)
    q = rnd(x @ wq.T).reshape(S, n_q_heads, d)
    k = rnd(x @ wk.T).reshape(S, n_kv_heads, d)
    v = rnd(x @ wv.T).reshape(S, n_kv_heads, d)
    out, lse = attention_forward(q, k, v, causal=causal)
    o = rnd(out)
    y = o.reshape(S, n_q_heads * d) @ wo.T
    return y, out, lse


def attention_block_rows(x, wq, wk, wv, wo, n_q_heads: int, n_kv_heads: int, rows, causal: bool = True):
    """y, out and lse of the block at selected query rows: k and v over the
    whole sequence (every row's keys), q only at ``rows``, the attention rows
    from :func:`oracle.attention.forward_rows`. The same numbers as
    :func:`attention_block_forward` at those rows, at O(S*d) attention work
    per row. Returns (y [R, Dm], out [R, Hq, d], lse [Hq, R])."""
    x, wq, wk, wv, wo = (np.asarray(t, dtype=np.float64) for t in (x, wq, wk, wv, wo))
    rows = np.asarray(rows, dtype=np.int64)
    S, Dm = x.shape
    d = wq.shape[0] // n_q_heads
    k = round_bf16(x @ wk.T).reshape(S, n_kv_heads, d)
    v = round_bf16(x @ wv.T).reshape(S, n_kv_heads, d)
    q = round_bf16(x[rows] @ wq.T).reshape(len(rows), n_q_heads, d)
    out, lse = forward_rows(q, k, v, rows, causal=causal)
    y = round_bf16(out).reshape(len(rows), n_q_heads * d) @ wo.T
    return y, out, lse


def attention_block_backward(x, wq, wk, wv, wo, dy, n_q_heads: int, n_kv_heads: int, causal: bool = True,
                             round_intermediates: bool = True):
    """Gradients of sum(dy * y) for the block of :func:`attention_block_forward`
    with respect to x and the four weights: (dx [S, Dm], dwq [Hq*d, Dm],
    dwk, dwv [Hkv*d, Dm], dwo [Dm, Hq*d]), all fp64."""
    x, wq, wk, wv, wo, dy = (np.asarray(t, dtype=np.float64) for t in (x, wq, wk, wv, wo, dy))
    S, Dm = x.shape
    d = wq.shape[0] // n_q_heads
    rnd = round_bf16 if round_intermediates else (lambda t: t)
    q = rnd(x @ wq.T).reshape(S, n_q_heads, d)
    k = rnd(x @ wk.T).reshape(S, n_kv_heads, d)
    v = rnd(x @ wv.T).reshape(S, n_kv_heads, d)
    out, _ = attention_forward(q, k, v, causal=causal)
    o = rnd(out).reshape(S, n_q_heads * d)
    # y = o Wo^T: the gradient reaches o through Wo and Wo through o
    dwo = dy.T @ o
    do = (dy @ wo).reshape(S, n_q_heads, d)
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal)
    dq = dq.reshape(S, n_q_heads * d)
    dk = dk.reshape(S, n_kv_heads * d)
    dv = dv.reshape(S, n_kv_heads * d)
    # q = x Wq^T (and k, v likewise): x collects every projection's share
    dx = dq @ wq + dk @ wk + dv @ wv
    return dx, dq.T @ x, dk.T @ x, dv.T @ x, dwo
