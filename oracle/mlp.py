"""Plain fp64 CPU oracle of the SwiGLU MLP that the sequence-tiled kernels
compute, forward and backward.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it, and it shares nothing with the HIP library.

Source: "Road to 5 Million Tokens: Breaking Barriers in Long Context
Training" talk summary, Chapters: the sequence-tiling chapter (the MLP, like
the loss, is computed in pieces along the sequence so that its S-long
intermediates never exist at once). Tiling changes only where those
intermediates are held, so this module writes the MLP out over the whole
sequence at once. The pages do not say which MLP; the reading taken is the
SwiGLU MLP of the Llama models the talk trains (torch Linear weights
[out, in], no biases):

    g = x Wg^T,  u = x Wu^T,  a = silu(g) * u,  y = a Wd^T,  silu(z) = z sigmoid(z)
  backward, given dy:
    da = dy Wd,  du = da * silu(g),  dg = da * u * silu'(g),
    silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
    dx = dg Wg + du Wu,  dWg = dg^T x,  dWu = du^T x,  dWd = dy^T a

g, u, a and y are the bf16 tensors a bf16 layer hands on: each is rounded
(float32, then bf16, nearest even) where it is formed, and the gradients are
taken through those values (the rounding passes gradients straight through).
"""

from __future__ import annotations

import numpy as np

from .block import round_bf16

__all__ = ["swiglu_mlp"]


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def swiglu_mlp(x, wg, wu, wd, dy=None):
    """y [S, Dm] (and, given dy, (dx, dWg, dWu, dWd)) in float64."""
    x, wg, wu, wd = (np.asarray(t, dtype=np.float64) for t in (x, wg, wu, wd))
    g = round_bf16(x @ wg.T)
    u = round_bf16(x @ wu.T)
    sg = _sigmoid(g)
    a = round_bf16(g * sg * u)
    y = round_bf16(a @ wd.T)
    if dy is None:
        return y
    dy = np.asarray(dy, dtype=np.float64)
    da = dy @ wd
    du = da * g * sg
    dg = da * u * sg * (1.0 + g * (1.0 - sg))
    dx = dg @ wg + du @ wu
    return y, (dx, dg.T @ x, du.T @ x, dy.T @ a)
