"""The oracle on random shapes and document splits (no GPU).

Hypothesis draws the sequence length, the query and kv head counts, the head
dim, the oracle's row block, causal or not, and packed-document offsets (empty
and length-one documents included). The full-tensor oracle must match torch's
float64 scaled_dot_product_attention with the explicit allowed-keys mask, and
its autograd, in out, lse, dq, dk and dv. The O(S*d)-per-row and per-key
functions that the large-size GPU checks rely on must match the full-tensor
ones on random samples of rows and keys.
"""

import math

import numpy as np
import torch
import torch.nn.functional as F
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle.attention as oracle
from oracle_pins import _doc_allowed


@st.composite
def cases(draw):
    S = draw(st.integers(1, 48))
    Hkv = draw(st.integers(1, 3))
    G = draw(st.integers(1, 3))
    d = draw(st.integers(1, 12))
    causal = draw(st.booleans())
    block = draw(st.integers(1, 20))
    docs = None
    if draw(st.booleans()):
        cuts = draw(st.lists(st.integers(0, S), max_size=4))
        docs = [0] + sorted(cuts) + [S]
    seed = draw(st.integers(0, 2**31 - 1))
    return S, Hkv * G, Hkv, d, causal, block, docs, seed


def _inputs(S, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((S, Hq, d)), rng.standard_normal((S, Hkv, d)), rng.standard_normal((S, Hkv, d)),
            rng.standard_normal((S, Hq, d)))


def _allowed(S, causal, docs):
    if docs is None:
        return np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
    return _doc_allowed(S, docs, causal)


@settings(max_examples=150, deadline=None, derandomize=True)
@given(cases())
def test_full_tensor_oracle_matches_torch_sdpa_and_autograd(c):
    S, Hq, Hkv, d, causal, block, docs, seed = c
    q, k, v, do = _inputs(S, Hq, Hkv, d, seed)
    out, lse = oracle.attention_forward(q, k, v, causal=causal, block=block, doc_offsets=docs)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=causal, block=block, doc_offsets=docs)

    G = Hq // Hkv
    mask = torch.tensor(_allowed(S, causal, docs))
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    qh = tq.permute(1, 0, 2).unsqueeze(0)
    kh = tk.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
    vh = tv.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask).squeeze(0).permute(1, 0, 2)
    np.testing.assert_allclose(out, o.detach().numpy(), rtol=1e-11, atol=1e-12)
    sc = (qh[0] @ kh[0].transpose(1, 2)) / math.sqrt(d)
    ref_lse = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1).detach().numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-11, atol=1e-12)
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)


@settings(max_examples=150, deadline=None, derandomize=True)
@given(cases(), st.data())
def test_row_and_key_functions_match_the_full_tensor_oracle(c, data):
    S, Hq, Hkv, d, causal, block, docs, seed = c
    q, k, v, do = _inputs(S, Hq, Hkv, d, seed)
    out, lse = oracle.attention_forward(q, k, v, causal=causal, block=block, doc_offsets=docs)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=causal, block=block, doc_offsets=docs)

    rows = np.array(data.draw(st.lists(st.integers(0, S - 1), min_size=1, max_size=6, unique=True)))
    o_r, l_r = oracle.forward_rows(q[rows], k, v, rows, causal=causal, doc_offsets=docs)
    np.testing.assert_allclose(o_r, out[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_r, lse[:, rows], rtol=1e-12, atol=1e-13)
    dq_r = oracle.backward_rows_dq(q[rows], k, v, do[rows], rows, causal=causal, doc_offsets=docs)
    np.testing.assert_allclose(dq_r, dq[rows], rtol=1e-10, atol=1e-12)
    o_f, l_f, dq_f = oracle.rows_forward_dq(q[rows], k, v, do[rows], rows, causal=causal, doc_offsets=docs)
    np.testing.assert_allclose(o_f, out[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_f, lse[:, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dq_f, dq[rows], rtol=1e-10, atol=1e-12)

    cols = np.array(data.draw(st.lists(st.integers(0, S - 1), min_size=1, max_size=6, unique=True)))
    dk_c, dv_c = oracle.backward_cols_dkdv(q, k, v, do, cols, causal=causal, doc_offsets=docs)
    np.testing.assert_allclose(dk_c, dk[cols], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv_c, dv[cols], rtol=1e-10, atol=1e-12)
    # the rows those keys need: the contiguous range from the first to the last
    # row that may attend to one of them
    need = oracle.cols_rows_needed(cols, S, causal=causal, doc_offsets=docs)
    reach = [i for i in range(S) if _allowed(S, causal, docs)[i, cols].any()]
    assert list(need) == list(range(reach[0], reach[-1] + 1))
