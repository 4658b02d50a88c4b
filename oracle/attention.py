"""Plain, slow fp64 CPU oracle of exact causal GQA attention, forward and backward.

TEST INFRASTRUCTURE ONLY. This module is the checker of the HIP path, not a
part of it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code, header,
table or helper with the HIP library and imports nothing from it.

Sources (web pages, cited by title and section):

[ROAD]  "Road to 5 Million Tokens: Breaking Barriers in Long Context Training"
        (Max Ryabinin, AI Engineer Europe 2026), talk summary page: sections
        "Chapters" (the DeepSpeed Ulysses chapter, the chapter on processing
        heads in batches, the Q&A chapter) and "Glossary" (UPipe, Ulysses).
[DIGEST] Russian digest of the same talk (transcript digest page): "Quiz"
        answers on Ulysses and on U-Pipe; "Insights" 02.
[MAXTEXT] Article on long-context training in MaxText v0.2.4 on Cloud TPU:
        the release section (attention variants MHA / GQA / MLA; Splash skips
        fully masked blocks), the section on where long-sequence training gets
        stuck (each position looks back over all earlier positions), the
        strategy-choice table (Ulysses splits heads, not positions), and the
        note that several samples packed into one long sequence need no
        padding under Splash attention.

What the oracle computes. Under Ulysses-style context parallelism a GPU runs
exact attention for its own heads over the whole sequence [ROAD Chapters,
Ulysses; DIGEST Quiz, Ulysses]. UPipe only changes *when* those heads run
(sequential head chunks reusing one buffer) [ROAD Chapters, batched heads;
DIGEST Quiz, U-Pipe]; it does not change what each head computes. Nothing is
approximated, so this module writes the definition of attention out, in
float64, with every input taken as the exact value of its element:

    A(i)   = {0..i} if causal else {0..S-1}            (look-back set)
             intersected, for packed sequences, with doc(i) = the positions
             of the document that holds i [MAXTEXT, packing note]
    s_ij   = tau * <q_hi, k_gj>,  tau = 1/sqrt(d),  g = kv head of h
    LSE_hi = log sum_{j in A(i)} exp(s_ij)             (natural log)
    P_ij   = exp(s_ij - LSE_hi)
    O_hi   = sum_{j in A(i)} P_ij v_gj
  backward, given the upstream gradient dO:
    D_hi   = <dO_hi, O_hi>
    dP_ij  = <dO_hi, v_gj>
    dS_ij  = P_ij (dP_ij - D_hi)
    dQ_hi  = tau sum_j dS_ij k_gj
    dK_gj  = tau sum_{h in group g} sum_{i: j in A(i)} dS_ij q_hi
    dV_gj  = sum_{h in group g} sum_{i: j in A(i)} P_ij dO_hi

Readings where the pages are silent or ambiguous:
  * causal look-back includes the position itself (j <= i);
  * tau = 1/sqrt(d); LSE is a natural log;
  * GQA heads are grouped contiguously: q head h reads kv head h // (Hq/Hkv);
  * layouts: q, k, v, dO, O are [S, H, d] (token-major); LSE is [Hq, S];
  * packed documents are contiguous runs of positions given by offsets
    0 = o_0 <= o_1 <= ... <= o_n = S (document m holds o_m .. o_{m+1}-1;
    empty documents are allowed); a position attends only within its own
    document, and causally within it when causal.

Algorithm: row blocks of R query rows; for each block the full score rows are
formed, then (1) the row max, (2) exp and row sum, (3) the weighted sum of V.
No online softmax, no tiling of the key axis. numpy matmul is the only library
primitive used.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "kv_head_of",
    "attention_forward",
    "attention_backward",
    "forward_rows",
    "backward_rows_dq",
    "rows_forward_dq",
    "backward_cols_dkdv",
    "cols_rows_needed",
    "document_bounds",
]

# Upper bound on the number of float64 score elements held at once (1 GiB).
# Batching only: each batch of rows streams K and V once, so larger batches
# read them fewer times; the numbers do not depend on it.
_SCORE_BUDGET = 1 << 27


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head read by query head ``h`` under GQA (contiguous groups)."""
    if n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of kv heads")
    return h // (n_q_heads // n_kv_heads)


def document_bounds(doc_offsets, S: int):
    """(first, last): for every position i, the first and the last position of
    the document that holds i, from offsets o_0 = 0 <= ... <= o_n = S."""
    off = np.asarray(doc_offsets, dtype=np.int64)
    if off.ndim != 1 or len(off) < 2 or off[0] != 0 or off[-1] != S or np.any(np.diff(off) < 0):
        raise ValueError("document offsets must rise from 0 to S")
    doc = np.searchsorted(off, np.arange(S), side="right") - 1  # last m with o_m <= i
    return off[doc], off[doc + 1] - 1


def _look_back_mask(rows: np.ndarray, n_cols: int, causal: bool, bounds=None) -> np.ndarray | None:
    """True where key j is NOT in A(i) for each row i in ``rows``."""
    mask = None
    if causal:
        mask = np.arange(n_cols)[None, :] > rows[:, None]
    if bounds is not None:
        first, last = bounds
        cols = np.arange(n_cols)[None, :]
        outside = (cols < first[rows][:, None]) | (cols > last[rows][:, None])
        mask = outside if mask is None else (mask | outside)
    return mask


def _bounds(doc_offsets, S):
    return None if doc_offsets is None else document_bounds(doc_offsets, S)


def _softmax_rows(s: np.ndarray):
    """Max, exp and sum along the last (key) axis of a score block (masked
    entries are -inf). Returns (P, LSE)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


def attention_forward(q, k, v, causal: bool = True, block: int = 256, doc_offsets=None):
    """Full-tensor forward. Returns (out [S,Hq,d], lse [Hq,S]) in float64.

    ``doc_offsets`` (optional) splits the sequence into packed documents."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    tau = 1.0 / math.sqrt(d)
    bounds = _bounds(doc_offsets, S)
    out = np.zeros((S, Hq, d))
    lse = np.zeros((Hq, S))
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        for r0 in range(0, S, block):
            r1 = min(S, r0 + block)
            rows = np.arange(r0, r1)
            n_cols = r1 if causal else S
            s = tau * (q[r0:r1, h, :] @ k[:n_cols, g, :].T)
            mask = _look_back_mask(rows, n_cols, causal, bounds)
            if mask is not None:
                s[mask] = -np.inf
            p, lse_blk = _softmax_rows(s)
            out[r0:r1, h, :] = p @ v[:n_cols, g, :]
            lse[h, r0:r1] = lse_blk
    return out, lse


def attention_backward(q, k, v, dout, causal: bool = True, block: int = 256, doc_offsets=None):
    """Full-tensor backward. Returns (dq, dk, dv) in float64, shaped like q, k, v.

    P is recomputed from the exact forward's LSE; D uses the exact O.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    tau = 1.0 / math.sqrt(d)
    bounds = _bounds(doc_offsets, S)
    out, lse = attention_forward(q, k, v, causal, block, doc_offsets)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        for r0 in range(0, S, block):
            r1 = min(S, r0 + block)
            rows = np.arange(r0, r1)
            n_cols = r1 if causal else S
            q_blk = q[r0:r1, h, :]
            do_blk = dout[r0:r1, h, :]
            s = tau * (q_blk @ k[:n_cols, g, :].T)
            mask = _look_back_mask(rows, n_cols, causal, bounds)
            if mask is not None:
                s[mask] = -np.inf
            p = np.exp(s - lse[h, r0:r1][:, None])
            dp = do_blk @ v[:n_cols, g, :].T
            D = (do_blk * out[r0:r1, h, :]).sum(axis=1)
            ds = p * (dp - D[:, None])
            dq[r0:r1, h, :] = tau * (ds @ k[:n_cols, g, :])
            dk[:n_cols, g, :] += tau * (ds.T @ q_blk)
            dv[:n_cols, g, :] += p.T @ do_blk
    return dq, dk, dv


def _row_batches(rows: np.ndarray, S: int, causal: bool, heads: int = 1):
    """Split sorted row indices into batches whose score block (rows x heads x
    keys) fits the budget."""
    order = np.argsort(rows, kind="stable")
    start, n = 0, len(order)
    while start < n:
        end = start + 1
        while end < n:
            width = int(rows[order[end]]) + 1 if causal else S
            if (end - start + 1) * heads * width > _SCORE_BUDGET:
                break
            end += 1
        yield order[start:end]
        start = end


def _group_scores(q_blk, k_g, tau, mask):
    """tau * <q, k> for a batch of rows and every query head of one kv group.

    q_blk [R, G, d], k_g [n, d] -> scores [R, G, n], with -inf where ``mask``
    [R, n] says the key is outside the row's look-back set.
    """
    R, G, d = q_blk.shape
    s = (tau * (q_blk.reshape(R * G, d) @ k_g.T)).reshape(R, G, -1)
    if mask is not None:
        s[np.broadcast_to(mask[:, None, :], s.shape)] = -np.inf
    return s


def _rows_matmul(a, b):
    """[R, G, n] @ [n, m] -> [R, G, m] as one 2-D matrix product."""
    R, G, n = a.shape
    return (a.reshape(R * G, n) @ b).reshape(R, G, b.shape[1])


def forward_rows(q_rows, k, v, rows, causal: bool = True, doc_offsets=None):
    """Exact O and LSE at selected query rows, O(S*d) work per row.

    ``q_rows`` [R,Hq,d] holds the query vectors of positions ``rows``. The
    query heads that share a kv head are scored together against it.
    Returns (out_rows [R,Hq,d], lse_rows [Hq,R]) in float64, in ``rows`` order.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    S, Hkv, d = k.shape
    Hq = q_rows.shape[1]
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    bounds = _bounds(doc_offsets, S)
    out = np.zeros((len(rows), Hq, d))
    lse = np.zeros((Hq, len(rows)))
    for sel in _row_batches(rows, S, causal, G):
        r = rows[sel]
        n_cols = int(r.max()) + 1 if causal else S
        mask = _look_back_mask(r, n_cols, causal, bounds)
        for g in range(Hkv):
            hs = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            s = _group_scores(q_rows[sel][:, hs, :], k[:n_cols, g, :], tau, mask)
            p, lse_blk = _softmax_rows(s)
            out[np.ix_(sel, hs)] = _rows_matmul(p, v[:n_cols, g, :])
            lse[np.ix_(hs, sel)] = lse_blk.T
    return out, lse


def backward_rows_dq(q_rows, k, v, dout_rows, rows, causal: bool = True, doc_offsets=None):
    """Exact dQ at selected query rows, O(S*d) work per row.

    ``q_rows`` and ``dout_rows`` [R,Hq,d] hold q and dO at positions ``rows``.
    D_hi needs only row i's own O, so each row is self-contained.
    Returns dq_rows [R,Hq,d] in float64, in ``rows`` order.
    """
    q_rows, k, v, dout_rows = _f64(q_rows), _f64(k), _f64(v), _f64(dout_rows)
    rows = np.asarray(rows, dtype=np.int64)
    S, Hkv, d = k.shape
    Hq = q_rows.shape[1]
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    bounds = _bounds(doc_offsets, S)
    dq = np.zeros((len(rows), Hq, d))
    for sel in _row_batches(rows, S, causal, G):
        r = rows[sel]
        n_cols = int(r.max()) + 1 if causal else S
        mask = _look_back_mask(r, n_cols, causal, bounds)
        for g in range(Hkv):
            hs = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            s = _group_scores(q_rows[sel][:, hs, :], k[:n_cols, g, :], tau, mask)
            p, _ = _softmax_rows(s)
            o = _rows_matmul(p, v[:n_cols, g, :])
            do_blk = dout_rows[sel][:, hs, :]
            D = (do_blk * o).sum(axis=-1)
            dp = _rows_matmul(do_blk, v[:n_cols, g, :].T)
            ds = p * (dp - D[..., None])
            dq[np.ix_(sel, hs)] = tau * _rows_matmul(ds, k[:n_cols, g, :])
    return dq


def rows_forward_dq(q_rows, k, v, dout_rows, rows, causal: bool = True, doc_offsets=None):
    """Exact O, LSE and dQ at selected query rows from one pass over each
    row's scores: the forward's softmax rows P and O = P V, then D = <dO, O>,
    dP = dO V^T, dS = P (dP - D) and dQ = tau dS K on the same P. O(S*d) work
    per row; the same numbers as :func:`forward_rows` and
    :func:`backward_rows_dq`, at two thirds of their combined cost.

    Returns (out_rows [R,Hq,d], lse_rows [Hq,R], dq_rows [R,Hq,d]) in float64,
    in ``rows`` order.
    """
    q_rows, k, v, dout_rows = _f64(q_rows), _f64(k), _f64(v), _f64(dout_rows)
    rows = np.asarray(rows, dtype=np.int64)
    S, Hkv, d = k.shape
    Hq = q_rows.shape[1]
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    bounds = _bounds(doc_offsets, S)
    out = np.zeros((len(rows), Hq, d))
    lse = np.zeros((Hq, len(rows)))
    dq = np.zeros((len(rows), Hq, d))
    for sel in _row_batches(rows, S, causal, G):
        r = rows[sel]
        n_cols = int(r.max()) + 1 if causal else S
        mask = _look_back_mask(r, n_cols, causal, bounds)
        for g in range(Hkv):
            hs = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            k_g, v_g = k[:n_cols, g, :], v[:n_cols, g, :]
            s = _group_scores(q_rows[sel][:, hs, :], k_g, tau, mask)
            p, lse_blk = _softmax_rows(s)
            o = _rows_matmul(p, v_g)
            out[np.ix_(sel, hs)] = o
            lse[np.ix_(hs, sel)] = lse_blk.T
            do_blk = dout_rows[sel][:, hs, :]
            D = (do_blk * o).sum(axis=-1)
            ds = p * (_rows_matmul(do_blk, v_g.T) - D[..., None])
            dq[np.ix_(sel, hs)] = tau * _rows_matmul(ds, k_g)
    return out, lse, dq


def cols_rows_needed(cols, S: int, causal: bool = True, doc_offsets=None) -> np.ndarray:
    """The contiguous range of query rows from the first to the last row whose
    softmax reaches any of the keys ``cols``: from the first key on when causal
    (from 0 otherwise), narrowed to the keys' documents when the sequence is
    packed. Rows inside the range that reach none of the keys (possible with
    packed documents) add nothing to those keys' gradients. Sorted positions."""
    cols = np.asarray(cols, dtype=np.int64)
    bounds = _bounds(doc_offsets, S)
    first = int(cols.min()) if causal else 0
    end = S
    if bounds is not None:
        first = max(first, int(bounds[0][cols].min()))
        end = int(bounds[1][cols].max()) + 1
    return np.arange(first, end)


def backward_cols_dkdv(q, k, v, dout, cols, causal: bool = True, doc_offsets=None, row_stats=None):
    """Exact dK and dV at selected key rows, from the inputs alone.

    Key j collects from every row i with j in A(i): i >= j when causal, every
    row otherwise, and with packed documents only rows of j's own document.
    Each such row's LSE and O come from :func:`forward_rows`, so the cost is
    O(|rows| * S * d), which is small when the keys lie near the end of a
    causal sequence or in short documents. ``row_stats`` may hand in that
    step's result, (out [R,Hq,d], lse [Hq,R]) of :func:`forward_rows` at the
    rows :func:`cols_rows_needed` names, computed elsewhere (e.g. in pieces).
    Returns (dk_cols [C,Hkv,d], dv_cols [C,Hkv,d]).
    """
    k, v = _f64(k), _f64(v)
    cols = np.asarray(cols, dtype=np.int64)
    S, Hkv, d = k.shape
    Hq = q.shape[1]
    tau = 1.0 / math.sqrt(d)
    bounds = _bounds(doc_offsets, S)
    need = cols_rows_needed(cols, S, causal, doc_offsets)
    first, end = int(need[0]), int(need[-1]) + 1
    q_need, do_need = _f64(q[first:end]), _f64(dout[first:end])
    if row_stats is None:
        o_need, lse_need = forward_rows(q_need, k, v, need, causal, doc_offsets)
    else:
        o_need, lse_need = _f64(row_stats[0]), _f64(row_stats[1])
    dk = np.zeros((len(cols), Hkv, d))
    dv = np.zeros((len(cols), Hkv, d))
    n_rows = len(need)
    per = max(1, _SCORE_BUDGET // max(1, n_rows))
    for c0 in range(0, len(cols), per):
        cj = cols[c0:c0 + per]
        # row i (absolute index need[t]) contributes to key j only if j in A(i)
        excluded = (need[None, :] < cj[:, None]) if causal else None
        if bounds is not None:
            other_doc = (bounds[0][need][None, :] > cj[:, None]) | (bounds[1][need][None, :] < cj[:, None])
            excluded = other_doc if excluded is None else (excluded | other_doc)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            qh = q_need[:, h, :]
            doh = do_need[:, h, :]
            s = tau * (k[cj, g, :] @ qh.T)  # [C, n_rows] = s_ij transposed
            p = np.exp(s - lse_need[h][None, :])
            if excluded is not None:
                p[excluded] = 0.0
            D = (doh * o_need[:, h, :]).sum(axis=1)
            dp = v[cj, g, :] @ doh.T
            ds = p * (dp - D[None, :])
            dk[c0:c0 + per, g, :] += tau * (ds @ qh)
            dv[c0:c0 + per, g, :] += p @ doh
    return dk, dv
