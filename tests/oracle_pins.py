"""Pins that tie the CPU oracle to something other than itself.

Each pin takes an oracle *module* (the real ``oracle.attention`` or a copy
with a planted mistake) and raises AssertionError when the oracle disagrees
with: a library routine (torch's fp64 scaled_dot_product_attention and its
autograd), central finite differences, a closed form, or an identity that the
mathematics of softmax attention fixes. None of them retypes the oracle's
formulas.
"""

from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

RNG_SEED = 1234


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, causal):
    """torch fp64 SDPA on [S,H,d] arrays with contiguous GQA groups."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    tq = torch.tensor(q).permute(1, 0, 2).unsqueeze(0)
    tk = torch.tensor(k).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
    tv = torch.tensor(v).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
    return tq, tk, tv


def pin_sdpa_forward(mod, S=37, Hq=4, Hkv=2, d=16, causal=True):
    q, k, v = _rand((S, Hq, d), 1), _rand((S, Hkv, d), 2), _rand((S, Hkv, d), 3)
    out, lse = mod.attention_forward(q, k, v, causal=causal, block=8)
    tq, tk, tv = _sdpa(q, k, v, causal)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    ref = ref.squeeze(0).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # LSE: log of the softmax denominator, from a library logsumexp
    s = torch.einsum("hid,hjd->hij", tq[0], tk[0]) / math.sqrt(d)
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def pin_sdpa_backward(mod, S=29, Hq=4, Hkv=2, d=8, causal=True):
    q, k, v = _rand((S, Hq, d), 4), _rand((S, Hkv, d), 5), _rand((S, Hkv, d), 6)
    do = _rand((S, Hq, d), 7)
    dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, block=8)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    G = Hq // Hkv
    o = F.scaled_dot_product_attention(
        tq.permute(1, 0, 2).unsqueeze(0),
        tk.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0),
        tv.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0),
        is_causal=causal,
    ).squeeze(0).permute(1, 0, 2)
    o.backward(torch.tensor(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)


def pin_finite_differences(mod, S=6, Hq=2, Hkv=1, d=3, causal=True, eps=1e-6):
    """Central differences of f = sum(dO * O) against the analytic gradients."""
    q, k, v = _rand((S, Hq, d), 8), _rand((S, Hkv, d), 9), _rand((S, Hkv, d), 10)
    do = _rand((S, Hq, d), 11)
    dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, block=4)

    def f(qq, kk, vv):
        o, _ = mod.attention_forward(qq, kk, vv, causal=causal, block=4)
        return float((do * o).sum())

    def f_with(name, xx):
        args = {"q": q, "k": k, "v": v}
        args[name] = xx
        return f(args["q"], args["k"], args["v"])

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num[idx] = (f_with(name, xp) - f_with(name, xm)) / (2 * eps)
        err = np.abs(num - g).max() / max(1e-12, np.abs(g).max())
        assert err < 1e-6, f"finite differences disagree on d{name}: rel {err:.2e}"


def pin_row0_closed_form(mod, S=11, Hq=3, Hkv=1, d=8):
    """Causal row 0 sees only key 0: O_0 = v_0 and LSE_0 = <q_0,k_0>/sqrt(d)."""
    q, k, v = _rand((S, Hq, d), 12), _rand((S, Hkv, d), 13), _rand((S, Hkv, d), 14)
    out, lse = mod.attention_forward(q, k, v, causal=True)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], v[0, 0], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[h, 0], q[0, h] @ k[0, 0] / math.sqrt(d), rtol=1e-14)


def pin_uniform_keys(mod, S=19, Hq=2, Hkv=1, d=8):
    """All keys equal: scores are constant along each row, so O_i is the mean of
    v_0..v_i and LSE_i = <q_i,c>/sqrt(d) + ln(i+1)."""
    q, v = _rand((S, Hq, d), 15), _rand((S, Hkv, d), 16)
    c = _rand((d,), 17)
    k = np.broadcast_to(c, (S, Hkv, d)).copy()
    out, lse = mod.attention_forward(q, k, v, causal=True, block=5)
    means = np.cumsum(v[:, 0, :], axis=0) / np.arange(1, S + 1)[:, None]
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h, :], means, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[h], q[:, h, :] @ c / math.sqrt(d) + np.log(np.arange(1, S + 1)),
                                   rtol=1e-12, atol=1e-13)
    # q = 0 gives the same uniform weights whatever the keys
    k2 = _rand((S, Hkv, d), 18)
    out0, lse0 = mod.attention_forward(np.zeros_like(q), k2, v, causal=True, block=7)
    np.testing.assert_allclose(out0[:, 0, :], means, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse0[0], np.log(np.arange(1, S + 1)), rtol=1e-12, atol=1e-13)


def pin_ones_values(mod, S=23, Hq=2, Hkv=2, d=4):
    """Softmax rows sum to one, so V = 1 gives O = 1 (causal and not)."""
    q, k = _rand((S, Hq, d), 19) * 3, _rand((S, Hkv, d), 20) * 3
    v = np.ones((S, Hkv, d))
    for causal in (True, False):
        out, _ = mod.attention_forward(q, k, v, causal=causal, block=6)
        np.testing.assert_allclose(out, 1.0, rtol=1e-13)


def pin_last_row_noncausal(mod, S=17, Hq=2, Hkv=1, d=8):
    """The last causal row sees every key, so it equals the non-causal row."""
    q, k, v = _rand((S, Hq, d), 21), _rand((S, Hkv, d), 22), _rand((S, Hkv, d), 23)
    oc, lc = mod.attention_forward(q, k, v, causal=True)
    on, ln = mod.attention_forward(q, k, v, causal=False)
    np.testing.assert_allclose(oc[-1], on[-1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lc[:, -1], ln[:, -1], rtol=1e-13)
    assert np.abs(oc[0] - on[0]).max() > 1e-3  # row 0 does differ


def pin_gradient_sums(mod, S=21, Hq=4, Hkv=2, d=8, causal=True):
    """sum_j dK_j = 0 (softmax is blind to a shift of every key) and
    sum_j dV_j = sum over the group's heads and all rows of dO (rows of P sum
    to one)."""
    q, k, v = _rand((S, Hq, d), 24), _rand((S, Hkv, d), 25), _rand((S, Hkv, d), 26)
    do = _rand((S, Hq, d), 27)
    _, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, block=5)
    G = Hq // Hkv
    for g in range(Hkv):
        np.testing.assert_allclose(dk[:, g, :].sum(axis=0), 0.0, atol=1e-12)
        ref = do[:, g * G:(g + 1) * G, :].sum(axis=(0, 1))
        np.testing.assert_allclose(dv[:, g, :].sum(axis=0), ref, rtol=1e-12, atol=1e-12)


def pin_key_shift(mod, S=15, Hq=2, Hkv=1, d=8):
    """k_j -> k_j + c adds a per-row constant to the scores: O, dQ, dK, dV are
    unchanged and LSE_i moves by <q_i,c>/sqrt(d)."""
    q, k, v = _rand((S, Hq, d), 28), _rand((S, Hkv, d), 29), _rand((S, Hkv, d), 30)
    do = _rand((S, Hq, d), 31)
    c = _rand((d,), 32)
    o1, l1 = mod.attention_forward(q, k, v)
    o2, l2 = mod.attention_forward(q, k + c, v)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, (q @ c).T / math.sqrt(d), rtol=1e-11, atol=1e-12)
    g1 = mod.attention_backward(q, k, v, do)
    g2 = mod.attention_backward(q, k + c, v, do)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


def pin_gqa_equals_repeated_mha(mod, S=13, Hq=6, Hkv=2, d=4):
    """GQA equals MHA with each kv head repeated over its group of Hq/Hkv
    consecutive query heads; dK/dV are the group sums of the MHA ones."""
    q, k, v = _rand((S, Hq, d), 33), _rand((S, Hkv, d), 34), _rand((S, Hkv, d), 35)
    do = _rand((S, Hq, d), 36)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    og, lg = mod.attention_forward(q, k, v)
    om, lm = mod.attention_forward(q, kr, vr)
    np.testing.assert_allclose(og, om, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lg, lm, rtol=1e-13, atol=1e-14)
    dqg, dkg, dvg = mod.attention_backward(q, k, v, do)
    dqm, dkm, dvm = mod.attention_backward(q, kr, vr, do)
    np.testing.assert_allclose(dqg, dqm, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dkg, dkm.reshape(S, Hkv, G, d).sum(axis=2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dvg, dvm.reshape(S, Hkv, G, d).sum(axis=2), rtol=1e-12, atol=1e-13)


def pin_sampled_functions(mod, S=53, Hq=4, Hkv=1, d=8):
    """The O(S*d)-per-row functions agree with the full-tensor ones (which the
    other pins tie to torch and to finite differences)."""
    q, k, v = _rand((S, Hq, d), 37), _rand((S, Hkv, d), 38), _rand((S, Hkv, d), 39)
    do = _rand((S, Hq, d), 40)
    for causal in (True, False):
        out, lse = mod.attention_forward(q, k, v, causal=causal, block=9)
        dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, block=9)
        # one sample with the last row, one that stays in the first half
        for rows in (np.array([0, 1, 7, 8, 31, 52, 20]), np.array([3, 0, 11, 25])):
            o_r, l_r = mod.forward_rows(q[rows], k, v, rows, causal=causal)
            np.testing.assert_allclose(o_r, out[rows], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l_r, lse[:, rows], rtol=1e-12, atol=1e-13)
            dq_r = mod.backward_rows_dq(q[rows], k, v, do[rows], rows, causal=causal)
            np.testing.assert_allclose(dq_r, dq[rows], rtol=1e-11, atol=1e-12)
            # the single-pass row function: the same O, LSE and dQ
            o_f, l_f, dq_f = mod.rows_forward_dq(q[rows], k, v, do[rows], rows, causal=causal)
            np.testing.assert_allclose(o_f, out[rows], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l_f, lse[:, rows], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(dq_f, dq[rows], rtol=1e-11, atol=1e-12)
        cols = np.array([52, 40, 45, 3]) if not causal else np.array([52, 40, 45])
        dk_c, dv_c = mod.backward_cols_dkdv(q, k, v, do, cols, causal=causal)
        np.testing.assert_allclose(dk_c, dk[cols], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dv_c, dv[cols], rtol=1e-11, atol=1e-12)
        # the rows the keys need, their forward computed in two pieces and handed in
        need = mod.cols_rows_needed(cols, S, causal=causal)
        assert list(need) == (list(range(40, S)) if causal else list(range(S)))
        h = len(need) // 2
        o1, l1 = mod.forward_rows(q[need[:h]], k, v, need[:h], causal=causal)
        o2, l2 = mod.forward_rows(q[need[h:]], k, v, need[h:], causal=causal)
        stats = (np.concatenate([o1, o2]), np.concatenate([l1, l2], axis=1))
        dk_s, dv_s = mod.backward_cols_dkdv(q, k, v, do, cols, causal=causal, row_stats=stats)
        np.testing.assert_allclose(dk_s, dk[cols], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dv_s, dv[cols], rtol=1e-11, atol=1e-12)


# --- packed documents -------------------------------------------------------
# Offsets with an empty document, a length-1 document, documents that end
# mid-way and one that runs to the end.
DOC_OFFSETS = [0, 1, 9, 9, 24, 30, 41]


def _doc_allowed(S, offsets, causal):
    """[S,S] booleans, True where row i may attend to key j: one square block
    per document, lower triangle when causal."""
    allowed = np.zeros((S, S), dtype=bool)
    for a, b in zip(offsets[:-1], offsets[1:]):
        allowed[a:b, a:b] = True
    if causal:
        allowed &= np.tril(np.ones((S, S), dtype=bool))
    return allowed


def pin_docs_sdpa(mod, S=41, Hq=4, Hkv=2, d=8):
    """Packed documents against torch's fp64 SDPA (and its autograd) with an
    explicit block-diagonal boolean mask."""
    q, k, v = _rand((S, Hq, d), 41), _rand((S, Hkv, d), 42), _rand((S, Hkv, d), 43)
    do = _rand((S, Hq, d), 44)
    G = Hq // Hkv
    for causal in (True, False):
        mask = torch.tensor(_doc_allowed(S, DOC_OFFSETS, causal))
        out, lse = mod.attention_forward(q, k, v, causal=causal, block=7, doc_offsets=DOC_OFFSETS)
        dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, block=7, doc_offsets=DOC_OFFSETS)
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        qh = tq.permute(1, 0, 2).unsqueeze(0)
        kh = tk.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
        vh = tv.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
        o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask).squeeze(0).permute(1, 0, 2)
        np.testing.assert_allclose(out, o.detach().numpy(), rtol=1e-12, atol=1e-12)
        sc = (qh[0] @ kh[0].transpose(1, 2)) / math.sqrt(d)
        ref_lse = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1).detach().numpy()
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
        o.backward(torch.tensor(do))
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)


def pin_docs_packed_equals_separate(mod, S=41, Hq=4, Hkv=1, d=8):
    """Packing is invisible: each document's rows and keys come out as if that
    document had been run alone (every output, causal and not)."""
    q, k, v = _rand((S, Hq, d), 45), _rand((S, Hkv, d), 46), _rand((S, Hkv, d), 47)
    do = _rand((S, Hq, d), 48)
    for causal in (True, False):
        out, lse = mod.attention_forward(q, k, v, causal=causal, block=6, doc_offsets=DOC_OFFSETS)
        grads = mod.attention_backward(q, k, v, do, causal=causal, block=6, doc_offsets=DOC_OFFSETS)
        for a, b in zip(DOC_OFFSETS[:-1], DOC_OFFSETS[1:]):
            if a == b:
                continue
            o1, l1 = mod.attention_forward(q[a:b], k[a:b], v[a:b], causal=causal, block=6)
            np.testing.assert_allclose(out[a:b], o1, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[:, a:b], l1, rtol=1e-12, atol=1e-13)
            g1 = mod.attention_backward(q[a:b], k[a:b], v[a:b], do[a:b], causal=causal, block=6)
            for x, y in zip(grads, g1):
                np.testing.assert_allclose(x[a:b], y, rtol=1e-11, atol=1e-12)


def pin_docs_single_is_plain(mod, S=29, Hq=2, Hkv=1, d=8):
    """One document spanning the sequence is the unpacked computation, exactly."""
    q, k, v = _rand((S, Hq, d), 49), _rand((S, Hkv, d), 50), _rand((S, Hkv, d), 51)
    do = _rand((S, Hq, d), 52)
    for causal in (True, False):
        a = mod.attention_forward(q, k, v, causal=causal, block=8, doc_offsets=[0, S])
        b = mod.attention_forward(q, k, v, causal=causal, block=8)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
        a = mod.attention_backward(q, k, v, do, causal=causal, block=8, doc_offsets=[0, S])
        b = mod.attention_backward(q, k, v, do, causal=causal, block=8)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def pin_docs_length_one(mod, S=13, Hq=4, Hkv=2, d=8):
    """Every document one position long: each row sees only itself, so
    O_i = v_i, LSE_i = <q_i,k_i>/sqrt(d), dQ = dK = 0 (P = 1 leaves dS = 0) and
    dV_j = the group's sum of dO_j."""
    q, k, v = _rand((S, Hq, d), 53), _rand((S, Hkv, d), 54), _rand((S, Hkv, d), 55)
    do = _rand((S, Hq, d), 56)
    G = Hq // Hkv
    offs = list(range(S + 1))
    for causal in (True, False):
        out, lse = mod.attention_forward(q, k, v, causal=causal, doc_offsets=offs)
        dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, doc_offsets=offs)
        for h in range(Hq):
            g = h // G
            np.testing.assert_allclose(out[:, h, :], v[:, g, :], rtol=0, atol=1e-15)
            np.testing.assert_allclose(lse[h], (q[:, h, :] * k[:, g, :]).sum(-1) / math.sqrt(d), rtol=1e-13)
        np.testing.assert_allclose(dq, 0.0, atol=1e-14)
        np.testing.assert_allclose(dk, 0.0, atol=1e-14)
        np.testing.assert_allclose(dv, do.reshape(S, Hkv, G, d).sum(axis=2), rtol=1e-13, atol=1e-14)


def pin_docs_sampled_functions(mod, S=41, Hq=4, Hkv=2, d=8):
    """The per-row and per-key functions agree with the full-tensor ones under
    packed documents."""
    q, k, v = _rand((S, Hq, d), 57), _rand((S, Hkv, d), 58), _rand((S, Hkv, d), 59)
    do = _rand((S, Hq, d), 60)
    for causal in (True, False):
        out, lse = mod.attention_forward(q, k, v, causal=causal, block=5, doc_offsets=DOC_OFFSETS)
        dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, block=5, doc_offsets=DOC_OFFSETS)
        rows = np.array([0, 1, 8, 9, 23, 24, 29, 30, 40, 15])
        o_r, l_r = mod.forward_rows(q[rows], k, v, rows, causal=causal, doc_offsets=DOC_OFFSETS)
        np.testing.assert_allclose(o_r, out[rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l_r, lse[:, rows], rtol=1e-12, atol=1e-13)
        dq_r = mod.backward_rows_dq(q[rows], k, v, do[rows], rows, causal=causal, doc_offsets=DOC_OFFSETS)
        np.testing.assert_allclose(dq_r, dq[rows], rtol=1e-11, atol=1e-12)
        o_f, l_f, dq_f = mod.rows_forward_dq(q[rows], k, v, do[rows], rows, causal=causal,
                                             doc_offsets=DOC_OFFSETS)
        np.testing.assert_allclose(o_f, out[rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l_f, lse[:, rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dq_f, dq[rows], rtol=1e-11, atol=1e-12)
        for cols in (np.array([40, 31, 25, 12]), np.array([0, 5]), np.array([29, 24])):
            dk_c, dv_c = mod.backward_cols_dkdv(q, k, v, do, cols, causal=causal, doc_offsets=DOC_OFFSETS)
            np.testing.assert_allclose(dk_c, dk[cols], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(dv_c, dv[cols], rtol=1e-11, atol=1e-12)
        # keys 29 and 24 sit in the document [24, 30): only its rows are needed
        need = mod.cols_rows_needed(np.array([29, 24]), S, causal=causal, doc_offsets=DOC_OFFSETS)
        assert list(need) == list(range(24, 30))


ALL_PINS = [
    pin_sdpa_forward,
    pin_sdpa_backward,
    pin_finite_differences,
    pin_row0_closed_form,
    pin_uniform_keys,
    pin_ones_values,
    pin_last_row_noncausal,
    pin_gradient_sums,
    pin_key_shift,
    pin_gqa_equals_repeated_mha,
    pin_sampled_functions,
    pin_docs_sdpa,
    pin_docs_packed_equals_separate,
    pin_docs_single_is_plain,
    pin_docs_length_one,
    pin_docs_sampled_functions,
]


def failing_pins(mod):
    """Names of the pins that ``mod`` fails (an exception of any kind counts)."""
    bad = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:  # noqa: BLE001 - a crash is a failed pin too
            bad.append(pin.__name__)
    return bad


# --- the attention block (projections around the chunked attention) ---------

def _bf16_values(shape, seed, scale=1.0):
    """Random values that bf16 holds exactly (a bf16 tensor's contents)."""
    t = torch.tensor(_rand(shape, seed) * scale).to(torch.bfloat16).to(torch.float64)
    return t.numpy()


def pin_round_bf16(bmod, amod=None):
    """round_bf16 against torch's float32 -> bfloat16 conversion (round to
    nearest even), on random values, exact ties and values bf16 holds."""
    x = np.concatenate([_rand(4096, 61) * 10.0 ** np.arange(-3, 5).repeat(512),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 0.0, -0.0])])
    ref = torch.tensor(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bmod.round_bf16(x), ref)
    v = _bf16_values(1000, 62)
    np.testing.assert_array_equal(bmod.round_bf16(v), v)


def pin_block_vs_torch(bmod, amod=None, S=37, Dm=24, Hq=4, Hkv=2, d=8):
    """The block against torch: F.linear for each projection, bfloat16
    conversion for the rounding, fp64 SDPA (GQA via repeated kv heads) for
    the attention."""
    x = _bf16_values((S, Dm), 63)
    wq, wk, wv = _bf16_values((Hq * d, Dm), 64, 0.3), _bf16_values((Hkv * d, Dm), 65, 0.3), \
        _bf16_values((Hkv * d, Dm), 66, 0.3)
    wo = _bf16_values((Dm, Hq * d), 67, 0.3)
    for causal in (True, False):
        y, out, lse = bmod.attention_block_forward(x, wq, wk, wv, wo, Hq, Hkv, causal=causal)
        rnd = lambda t: t.to(torch.float32).to(torch.bfloat16).to(torch.float64)  # noqa: E731
        tx = torch.tensor(x)
        q = rnd(F.linear(tx, torch.tensor(wq))).reshape(S, Hq, d).permute(1, 0, 2)
        k = rnd(F.linear(tx, torch.tensor(wk))).reshape(S, Hkv, d).permute(1, 0, 2)
        v = rnd(F.linear(tx, torch.tensor(wv))).reshape(S, Hkv, d).permute(1, 0, 2)
        o = F.scaled_dot_product_attention(q.unsqueeze(0), k.repeat_interleave(Hq // Hkv, 0).unsqueeze(0),
                                           v.repeat_interleave(Hq // Hkv, 0).unsqueeze(0), is_causal=causal)
        o = o.squeeze(0).permute(1, 0, 2)
        np.testing.assert_allclose(out, o.numpy(), rtol=1e-11, atol=1e-12)
        ref_y = F.linear(rnd(o).reshape(S, Hq * d), torch.tensor(wo)).numpy()
        np.testing.assert_allclose(y, ref_y, rtol=1e-10, atol=1e-11)


def pin_block_identity_is_attention(bmod, amod, S=29, Hq=4, Hkv=2, d=8):
    """With identity projections (Dm = Hq*d) the block is plain attention of
    slices of x, and y its output rounded to bf16."""
    Dm = Hq * d
    x = _bf16_values((S, Dm), 68)
    eye = np.eye(Dm)
    wq, wk, wv, wo = eye, eye[:Hkv * d], eye[Hkv * d:2 * Hkv * d], eye
    y, out, lse = bmod.attention_block_forward(x, wq, wk, wv, wo, Hq, Hkv)
    o_ref, l_ref = amod.attention_forward(x.reshape(S, Hq, d), x[:, :Hkv * d].reshape(S, Hkv, d),
                                          x[:, Hkv * d:2 * Hkv * d].reshape(S, Hkv, d))
    np.testing.assert_array_equal(out, o_ref)
    np.testing.assert_array_equal(lse, l_ref)
    np.testing.assert_array_equal(y, bmod.round_bf16(o_ref).reshape(S, Dm))


def pin_block_linear_in_wo_and_head_order(bmod, amod=None, S=23, Dm=16, Hq=4, Hkv=2, d=8):
    """y is linear in Wo, and relabelling query heads inside a kv group (rows
    of Wq and columns of Wo moved together) leaves y unchanged."""
    x = _bf16_values((S, Dm), 69)
    wq, wk, wv = _bf16_values((Hq * d, Dm), 70, 0.3), _bf16_values((Hkv * d, Dm), 71, 0.3), \
        _bf16_values((Hkv * d, Dm), 72, 0.3)
    wo1, wo2 = _bf16_values((Dm, Hq * d), 73, 0.3), _bf16_values((Dm, Hq * d), 74, 0.3)
    y1 = bmod.attention_block_forward(x, wq, wk, wv, wo1, Hq, Hkv)[0]
    y2 = bmod.attention_block_forward(x, wq, wk, wv, wo2, Hq, Hkv)[0]
    y12 = bmod.attention_block_forward(x, wq, wk, wv, wo1 + wo2, Hq, Hkv)[0]
    np.testing.assert_allclose(y12, y1 + y2, rtol=1e-12, atol=1e-12)
    perm = [1, 0, 3, 2]  # swaps heads inside each group of G = 2
    rows = np.concatenate([np.arange(h * d, (h + 1) * d) for h in perm])
    yp = bmod.attention_block_forward(x, wq[rows], wk, wv, wo1[:, rows], Hq, Hkv)[0]
    np.testing.assert_allclose(yp, y1, rtol=1e-12, atol=1e-12)


def pin_block_rows(bmod, amod=None, S=41, Dm=16, Hq=4, Hkv=2, d=8):
    """The sampled-row block function equals the full one at those rows."""
    x = _bf16_values((S, Dm), 75)
    wq, wk, wv = _bf16_values((Hq * d, Dm), 76, 0.3), _bf16_values((Hkv * d, Dm), 77, 0.3), \
        _bf16_values((Hkv * d, Dm), 78, 0.3)
    wo = _bf16_values((Dm, Hq * d), 79, 0.3)
    rows = np.array([0, 1, 17, 40, 22, 7])
    for causal in (True, False):
        y, out, lse = bmod.attention_block_forward(x, wq, wk, wv, wo, Hq, Hkv, causal=causal)
        yr, outr, lser = bmod.attention_block_rows(x, wq, wk, wv, wo, Hq, Hkv, rows, causal=causal)
        np.testing.assert_allclose(yr, y[rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(outr, out[rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lser, lse[:, rows], rtol=1e-12, atol=1e-13)


class _StraightThroughBf16(torch.autograd.Function):
    """bf16 rounding forward, identity backward (the gradient stays fp64)."""

    @staticmethod
    def forward(ctx, t):
        return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)

    @staticmethod
    def backward(ctx, grad):
        return grad


def _block_weights(S, Dm, Hq, Hkv, d, seed):
    x = _bf16_values((S, Dm), seed)
    wq, wk, wv = _bf16_values((Hq * d, Dm), seed + 1, 0.3), _bf16_values((Hkv * d, Dm), seed + 2, 0.3), \
        _bf16_values((Hkv * d, Dm), seed + 3, 0.3)
    wo = _bf16_values((Dm, Hq * d), seed + 4, 0.3)
    dy = _bf16_values((S, Dm), seed + 5)
    return x, wq, wk, wv, wo, dy


def pin_block_backward_vs_torch(bmod, amod=None, S=31, Dm=24, Hq=4, Hkv=2, d=8):
    """The block's gradients against torch autograd: F.linear projections,
    fp64 SDPA with the kv heads repeated for GQA, the bfloat16 conversion as
    the straight-through rounding of q, k, v and o; causal and not."""
    x, wq, wk, wv, wo, dy = _block_weights(S, Dm, Hq, Hkv, d, 101)
    rnd = _StraightThroughBf16.apply
    for causal in (True, False):
        grads = bmod.attention_block_backward(x, wq, wk, wv, wo, dy, Hq, Hkv, causal=causal)
        tx, tq, tk, tv, to = (torch.tensor(t, requires_grad=True) for t in (x, wq, wk, wv, wo))
        q = rnd(F.linear(tx, tq)).reshape(S, Hq, d).permute(1, 0, 2)
        k = rnd(F.linear(tx, tk)).reshape(S, Hkv, d).permute(1, 0, 2)
        v = rnd(F.linear(tx, tv)).reshape(S, Hkv, d).permute(1, 0, 2)
        o = F.scaled_dot_product_attention(q.unsqueeze(0), k.repeat_interleave(Hq // Hkv, 0).unsqueeze(0),
                                           v.repeat_interleave(Hq // Hkv, 0).unsqueeze(0), is_causal=causal)
        y = F.linear(rnd(o.squeeze(0).permute(1, 0, 2).reshape(S, Hq * d)), to)
        y.backward(torch.tensor(dy))
        for got, ref in zip(grads, (tx.grad, tq.grad, tk.grad, tv.grad, to.grad)):
            assert got.shape == tuple(ref.shape)
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def pin_block_backward_finite_differences(bmod, amod=None, S=7, Dm=6, Hq=2, Hkv=1, d=3, eps=1e-5):
    """Without the roundings the block is smooth: each gradient's inner
    product with a random direction equals the central difference of
    sum(dy * y) along it."""
    x, wq, wk, wv, wo, dy = _block_weights(S, Dm, Hq, Hkv, d, 111)
    params = [x, wq, wk, wv, wo]

    def f(ps):
        y = bmod.attention_block_forward(*ps, Hq, Hkv, round_intermediates=False)[0]
        return float((dy * y).sum())

    grads = bmod.attention_block_backward(*params, dy, Hq, Hkv, round_intermediates=False)
    rng = np.random.default_rng(112)
    for i, g in enumerate(grads):
        e = rng.standard_normal(params[i].shape)
        plus = [p + eps * e if j == i else p for j, p in enumerate(params)]
        minus = [p - eps * e if j == i else p for j, p in enumerate(params)]
        fd = (f(plus) - f(minus)) / (2 * eps)
        np.testing.assert_allclose(float((g * e).sum()), fd, rtol=1e-6, atol=1e-9)


BLOCK_PINS = [pin_round_bf16, pin_block_vs_torch, pin_block_identity_is_attention,
              pin_block_linear_in_wo_and_head_order, pin_block_rows, pin_block_backward_vs_torch,
              pin_block_backward_finite_differences]


def failing_block_pins(bmod, amod):
    bad = []
    for pin in BLOCK_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bmod, amod)
        except Exception:  # noqa: BLE001
            bad.append(pin.__name__)
    return bad



# --- the sequence-tiled cross-entropy -----------------------------------------

def pin_ce_vs_torch(lmod, S=53, Dm=16, V=40):
    """loss against torch's cross_entropy (fp64, no reduction, ignore_index
    -100), dh and dW against its autograd of sum(scale * loss)."""
    h, w = _rand((S, Dm), 81), _rand((V, Dm), 82) * 0.5
    labels = np.random.default_rng(83).integers(0, V, size=S)
    labels[[3, 17, 40]] = -100
    scale = 0.37
    loss, dh, dw = lmod.cross_entropy(h, w, labels, scale=scale, block=7)
    th, tw = torch.tensor(h, requires_grad=True), torch.tensor(w, requires_grad=True)
    ref = F.cross_entropy(F.linear(th, tw), torch.tensor(labels), reduction="none", ignore_index=-100)
    np.testing.assert_allclose(loss, ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    (scale * ref).sum().backward()
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-11, atol=1e-12)


def pin_ce_closed_forms(lmod, S=9, Dm=4, V=16):
    """W = 0: every logit is 0, so loss = ln V and G = scale (1/V - onehot);
    dW rows then sum (over the vocabulary) to zero, as softmax rows sum to 1."""
    h = _rand((S, Dm), 84)
    labels = np.arange(S) % V
    loss, dh, dw = lmod.cross_entropy(h, np.zeros((V, Dm)), labels, scale=2.0)
    np.testing.assert_allclose(loss, np.log(V), rtol=1e-14)
    np.testing.assert_allclose(dh, 0.0, atol=1e-15)
    onehot = np.eye(V)[labels]
    np.testing.assert_allclose(dw, 2.0 * (1.0 / V - onehot).T @ h, rtol=1e-12, atol=1e-13)
    w = _rand((V, Dm), 85)
    _, _, dw = lmod.cross_entropy(h, w, labels)
    np.testing.assert_allclose(dw.sum(axis=0), 0.0, atol=1e-12)


CE_PINS = [pin_ce_vs_torch, pin_ce_closed_forms]


def failing_ce_pins(lmod):
    bad = []
    for pin in CE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(lmod)
        except Exception:  # noqa: BLE001
            bad.append(pin.__name__)
    return bad



# --- the sequence-tiled SwiGLU MLP ---------------------------------------------

def pin_mlp_vs_torch(mmod, S=37, Dm=16, Fh=24):
    """The MLP and its gradients against torch: F.linear, F.silu, the
    bfloat16 conversion as the rounding step (wrapped so that its gradient
    passes straight through in fp64), autograd for dx and the weight
    gradients."""
    x = _bf16_values((S, Dm), 91)
    wg, wu = _bf16_values((Fh, Dm), 92, 0.4), _bf16_values((Fh, Dm), 93, 0.4)
    wd = _bf16_values((Dm, Fh), 94, 0.4)
    dy = _bf16_values((S, Dm), 95)
    y, (dx, dwg, dwu, dwd) = mmod.swiglu_mlp(x, wg, wu, wd, dy)

    class Rnd(torch.autograd.Function):
        """bf16 rounding forward, identity backward (the gradient stays fp64)."""

        @staticmethod
        def forward(ctx, t):
            return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)

        @staticmethod
        def backward(ctx, grad):
            return grad

    rnd = Rnd.apply
    tx = torch.tensor(x, requires_grad=True)
    tg, tu, td = (torch.tensor(w, requires_grad=True) for w in (wg, wu, wd))
    g, u = rnd(F.linear(tx, tg)), rnd(F.linear(tx, tu))
    ty = rnd(F.linear(rnd(F.silu(g) * u), td))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=0, atol=0)
    ty.backward(torch.tensor(dy))
    for got, ref in ((dx, tx.grad), (dwg, tg.grad), (dwu, tu.grad), (dwd, td.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def pin_mlp_closed_forms(mmod, S=9, Dm=8, Fh=16):
    """Wu = 0: u = 0, so y = 0, and dWg = dx-from-g = 0 (du = da * silu(g)
    remains); silu(0) = 0 makes Wg = 0 give y = 0 and du = 0."""
    x = _bf16_values((S, Dm), 96)
    w = _bf16_values((Fh, Dm), 97, 0.5)
    wd = _bf16_values((Dm, Fh), 98, 0.5)
    dy = _bf16_values((S, Dm), 99)
    y, (dx, dwg, dwu, dwd) = mmod.swiglu_mlp(x, w, np.zeros((Fh, Dm)), wd, dy)
    np.testing.assert_array_equal(y, 0.0)
    np.testing.assert_array_equal(dwg, 0.0)
    np.testing.assert_array_equal(dwd, 0.0)
    assert np.abs(dwu).max() > 0
    y, (dx, dwg, dwu, dwd) = mmod.swiglu_mlp(x, np.zeros((Fh, Dm)), w, wd, dy)
    np.testing.assert_array_equal(y, 0.0)
    np.testing.assert_array_equal(dwu, 0.0)
    assert np.abs(dwg).max() > 0


MLP_PINS = [pin_mlp_vs_torch, pin_mlp_closed_forms]


def failing_mlp_pins(mmod):
    bad = []
    for pin in MLP_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mmod)
        except Exception:  # noqa: BLE001
            bad.append(pin.__name__)
    return bad
