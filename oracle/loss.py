"""Plain fp64 CPU oracle of the token-level cross-entropy over the
vocabulary, the loss the sequence-tiled kernel computes.

TEST INFRASTRUCTURE ONLY, like ``oracle.attention``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it, and it shares nothing with the HIP library.

Source: "Road to 5 Million Tokens: Breaking Barriers in Long Context
Training" talk summary, Chapters: the sequence-tiling chapter (the loss and
the MLP are computed in pieces along the sequence so that their S-long
intermediates -- here the [S, V] logits -- never exist at once). Tiling
changes only where the logits are held, not what is computed, so this module
writes the definition out over the whole sequence at once:

    z_i      = W h_i                      (logits, W [V, Dm] in torch Linear layout)
    lse_i    = log sum_j exp(z_ij)
    loss_i   = lse_i - z_i[label_i]       (0 where label_i < 0: ignored)
    G_ij     = scale * (exp(z_ij - lse_i) - [j == label_i])   (0 on ignored rows)
    dh_i     = sum_j G_ij W_j ,   dW_j = sum_i G_ij h_i

Readings where the pages are silent: natural log; a negative label marks a
token without a target (no loss, no gradient); ``scale`` is the upstream
gradient of each token's loss (1/N for a mean over N counted tokens).
"""

from __future__ import annotations

import numpy as np

__all__ = ["cross_entropy"]


def cross_entropy(h, w, labels, scale: float = 1.0, block: int = 512):
    """(loss [S], dh [S, Dm], dW [V, Dm]) in float64 for h [S, Dm], w [V, Dm],
    labels [S] (int; < 0 ignored). Rows are processed in blocks of ``block``
    (batching only)."""
    h, w = np.asarray(h, dtype=np.float64), np.asarray(w, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    S = h.shape[0]
    loss = np.zeros(S)
    dh = np.zeros_like(h)
    dw = np.zeros_like(w)
    for r0 in range(0, S, block):
        r1 = min(S, r0 + block)
        z = h[r0:r1] @ w.T
        m = z.max(axis=1, keepdims=True)
        lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
        lab = labels[r0:r1]
        counted = lab >= 0
        rows = np.arange(r1 - r0)
        picked = z[rows, np.where(counted, lab, 0)]
        loss[r0:r1] = np.where(counted, lse - picked, 0.0)
        g = np.exp(z - lse[:, None])
        g[rows[counted], lab[counted]] -= 1.0
        g *= scale
        g[~counted] = 0.0
        dh[r0:r1] = g @ w
        dw += g.T @ h[r0:r1]
    return loss, dh, dw
