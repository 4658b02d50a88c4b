"""Packed documents: the HIP path vs the fp64 CPU oracle, through the C ABI
(upipe_attn_fwd_docs / upipe_attn_bwd_docs).

Full tensors at small sizes, with documents that are empty, one position
long, end on and off the kernels' tile edges, and span several tiles; outputs
must also be bit-identical across head_chunk. At 1,048,576 tokens the
checks run on sampled rows (document edges included) and on keys at the ends
of documents. Every case prints its shape before it runs.
"""

import numpy as np
import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import OracleJobs, assert_close, bit_equal, f64, grad_scale, interleaved_parts, run
from long_context_attention_upipe_amd.workloads import (WORKLOADS, custom, doc_boundary_rows, doc_offsets,
                                                        make_inputs, sample_rows)
from oracle.attention import attention_backward, attention_forward, backward_cols_dkdv, rows_forward_dq

pytestmark = pytest.mark.gpu

# S = 1000: a length-1 document first, edges at 63/64 (the forward's key
# tile) and 128-multiples nearby, an empty document, and a ragged tail.
RAGGED = [0, 1, 63, 64, 64, 200, 333, 700, 701, 1000]


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _docs_case(w, offsets, hcs, causal=True, check_bwd=True):
    dev = _dev()
    print(f"\n  case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} {w.dtype} causal={causal} hcs={hcs} "
          f"docs={len(offsets) - 1}", flush=True)
    q, k, v, do = make_inputs(w, device="cpu")
    ro, rl = attention_forward(f64(q), f64(k), f64(v), causal=causal, doc_offsets=offsets)
    if check_bwd:
        rdq, rdk, rdv = attention_backward(f64(q), f64(k), f64(v), f64(do), causal=causal, doc_offsets=offsets)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    offs = torch.tensor(offsets, dtype=torch.int32, device=dev)
    first = None
    for hc in hcs:
        print(f"   head_chunk={hc}", flush=True)
        r = run(qd, kd, vd, dod if check_bwd else None, hc, causal=causal, doc_offsets=offs)
        assert_close("out", f64(r["out"]), ro, w.dtype)
        assert_close("lse", f64(r["lse"]), rl, w.dtype)
        if check_bwd:
            gs = grad_scale(w)
            assert_close("dq", f64(r["dq"]), rdq, w.dtype, grad_scale=gs, per_item=True)
            assert_close("dk", f64(r["dk"]), rdk, w.dtype, grad_scale=gs, per_item=True)
            assert_close("dv", f64(r["dv"]), rdv, w.dtype, grad_scale=gs, per_item=True)
        if first is None:
            first = r
        else:
            for name in r:
                assert bit_equal(r[name], first[name]), f"{name} differs between head_chunk {hcs[0]} and {hc}"


def test_docs_bf16_causal_ragged():
    _docs_case(custom(1000, 4, 1, 128, "bf16", seed=201, dout_scaled=True), RAGGED, (1, 2, 4))


def test_docs_bf16_non_causal_ragged():
    _docs_case(custom(1000, 4, 1, 128, "bf16", seed=202, dout_scaled=True), RAGGED, (1, 4), causal=False)


@pytest.mark.parametrize("causal", [True, False])
def test_docs_fp32_head_dim_64_two_kv_heads(causal):
    _docs_case(custom(1000, 4, 2, 64, "fp32", seed=203), RAGGED, (1, 2, 4), causal=causal)


def test_docs_bf16_head_dim_64():
    _docs_case(custom(1000, 4, 2, 64, "bf16", seed=204, dout_scaled=True), RAGGED, (1, 2))


def test_docs_fp32_head_dim_128():
    _docs_case(custom(700, 2, 1, 128, "fp32", seed=205), [0, 5, 130, 131, 500, 700], (1, 2))


def test_docs_tile_aligned_and_long():
    """Edges on 128-row tiles, one document of several tiles."""
    _docs_case(custom(2048, 4, 1, 128, "bf16", seed=206, dout_scaled=True), [0, 128, 256, 1024, 2048], (1, 4))


def test_docs_many_short_seeded():
    """4099 positions in seeded documents of 1..300 positions."""
    rng = np.random.default_rng(207)
    offs = [0]
    while offs[-1] < 4099:
        offs.append(min(4099, offs[-1] + int(rng.integers(1, 301))))
    _docs_case(custom(4099, 4, 1, 128, "bf16", seed=207, dout_scaled=True), offs, (1, 4))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [True, False])
def test_single_document_is_the_plain_call_bit_for_bit(dtype, causal):
    dev = _dev()
    w = custom(777, 4, 1, 128 if dtype == "bf16" else 64, dtype, seed=208, dout_scaled=True)
    print(f"\n  case one document S={w.S} {dtype} causal={causal}", flush=True)
    q, k, v, do = (t.to(dev) for t in make_inputs(w, device="cpu"))
    a = run(q, k, v, do, 2, causal=causal)
    b = run(q, k, v, do, 2, causal=causal, doc_offsets=torch.tensor([0, w.S], dtype=torch.int32, device=dev))
    for name in a:
        assert bit_equal(a[name], b[name]), f"{name}: one document differs from the plain call"


def test_length_one_documents_closed_form():
    """Every document one position long: out = v exactly, lse_i = <q_i,k_i>/sqrt(d),
    dQ = dK = 0 and dV = the group's sum of dO."""
    dev = _dev()
    w = custom(300, 4, 1, 128, "bf16", seed=209, dout_scaled=True)
    print(f"\n  case length-1 documents S={w.S}", flush=True)
    q, k, v, do = make_inputs(w, device="cpu")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    offs = torch.arange(w.S + 1, dtype=torch.int32, device=dev)
    r = run(qd, kd, vd, dod, 4, doc_offsets=offs)
    for h in range(w.Hq):
        assert torch.equal(r["out"][:, h], vd[:, 0]), f"out[:, {h}] != v"
    lse_ref = (f64(q) * f64(k)).sum(-1).T / np.sqrt(w.d)
    assert_close("lse", f64(r["lse"]), lse_ref, "bf16")
    assert_close("dq", f64(r["dq"]), np.zeros(q.shape), "bf16")
    assert_close("dk", f64(r["dk"]), np.zeros(k.shape), "bf16")
    assert_close("dv", f64(r["dv"]), f64(do).sum(axis=1, keepdims=True), "bf16")


def test_bad_offsets_are_refused_on_the_device():
    dev = _dev()
    w = custom(64, 2, 1, 64, "bf16", seed=210)
    q, k, v, _ = (t.to(dev) if t is not None else None for t in make_inputs(w, device="cpu", need_dout=False))
    for bad in ([0, 40, 30, 64], [0, 63], [2, 64]):
        with pytest.raises(up.UpipeError, match="rise"):
            up.attention_forward(q, k, v, doc_offsets=torch.tensor(bad, dtype=torch.int32, device=dev))


@pytest.mark.slow
def test_llama8b_share_1m_docs_sampled():
    """1,048,576 tokens in 16 log-uniform documents (1K-256K): O, LSE and dQ at
    4096 sampled rows plus the edges of every document; dK and dV at keys in
    the last 64 positions of four documents; outputs bit-identical across
    head_chunk 1, 2, 4."""
    dev = _dev()
    w = WORKLOADS["llama8b_share_s1m_docs"]
    offsets = doc_offsets(w)
    print(f"\n  case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} docs={len(offsets) - 1}", flush=True)
    q, k, v, do = make_inputs(w, device=dev)
    offs_t = torch.from_numpy(offsets).to(dev)
    rows = np.union1d(sample_rows(w.S, 4096, seed=w.seed + 7), doc_boundary_rows(offsets, len(offsets), w.seed + 8))
    rows_t = torch.from_numpy(rows).to(dev)
    kc, vc = f64(k), f64(v)
    qr, dor = f64(q[rows_t]), f64(do[rows_t])
    q32, do32 = q.float().cpu().numpy(), do.float().cpu().numpy()
    ends = [int(offsets[m + 1]) for m in (0, 3, len(offsets) // 2, len(offsets) - 2)]
    with OracleJobs() as jobs:
        # host side, concurrent with the GPU runs below
        parts = interleaved_parts(len(rows), 64)
        rows_job = jobs.map(lambda p: rows_forward_dq(qr[p], kc, vc, dor[p], rows[p], doc_offsets=offsets), parts,
                            "rows (O, LSE, dQ)")
        keys_job = jobs.map(lambda end: backward_cols_dkdv(q32, kc, vc, do32, np.arange(end - 64, end, dtype=np.int64),
                                                           doc_offsets=offsets), ends, "keys at document ends")
        r = None
        for hc in w.head_chunks:
            print(f"   head_chunk={hc}", flush=True)
            cur = run(q, k, v, do, hc, doc_offsets=offs_t)
            if r is None:
                r = cur
            else:
                for name in cur:
                    assert bit_equal(cur[name], r[name]), f"{name}: head_chunk {hc} differs"
                del cur
        gs = grad_scale(w)
        o_ref, l_ref, dq_ref = np.empty_like(qr), np.empty((w.Hq, len(rows))), np.empty_like(qr)
        for p, (o, lse, dq) in zip(parts, jobs.gather(rows_job)):
            o_ref[p], l_ref[:, p], dq_ref[p] = o, lse, dq
        assert_close("out", f64(r["out"][rows_t]), o_ref, w.dtype, per_item=True)
        assert_close("lse", f64(r["lse"][:, rows_t]), l_ref, w.dtype)
        assert_close("dq", f64(r["dq"][rows_t]), dq_ref, w.dtype, grad_scale=gs, per_item=True)
        for end, (dk_ref, dv_ref) in zip(ends, jobs.gather(keys_job)):
            keys_t = torch.arange(end - 64, end, device=dev)
            assert_close("dk", f64(r["dk"][keys_t]), dk_ref, w.dtype, grad_scale=gs, per_item=True)
            assert_close("dv", f64(r["dv"][keys_t]), dv_ref, w.dtype, grad_scale=gs, per_item=True)


@pytest.mark.slow
def test_llama8b_share_1m_docs_non_causal_sampled():
    """1,048,576 tokens in 16 documents, non-causal (a position sees its whole
    document): O, LSE and dQ at 1024 sampled rows plus the edges of every
    document (each non-causal row costs its whole document in the oracle);
    dK and dV at 64 keys in each of the four shortest documents (without the
    causal mask a key's gradient takes every row of its document, so exact
    values stay cheap only in short ones). A document's results are those of
    the document run alone (pinned in the oracle's tests), so the keys' oracle
    runs on each document's slice. Outputs bit-identical across head_chunk 1,
    2, 4."""
    dev = _dev()
    w = WORKLOADS["llama8b_share_s1m_docs"]
    offsets = doc_offsets(w)
    print(f"\n  case {w.name} non-causal S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} docs={len(offsets) - 1}", flush=True)
    q, k, v, do = make_inputs(w, device=dev)
    offs_t = torch.from_numpy(offsets).to(dev)
    rows = np.union1d(sample_rows(w.S, 1024, seed=w.seed + 17), doc_boundary_rows(offsets, len(offsets), w.seed + 18))
    rows_t = torch.from_numpy(rows).to(dev)
    kc, vc = f64(k), f64(v)
    qr, dor = f64(q[rows_t]), f64(do[rows_t])
    lengths = np.diff(offsets)
    short = [(int(offsets[m]), int(offsets[m + 1])) for m in np.argsort(lengths, kind="stable")[:4]]
    q64, do64 = f64(q), f64(do)

    def doc_keys(span):
        start, end = span
        keys = np.arange(min(64, end - start), dtype=np.int64)
        return backward_cols_dkdv(q64[start:end], kc[start:end], vc[start:end], do64[start:end], keys, causal=False)

    with OracleJobs() as jobs:
        # host side, concurrent with the GPU runs below
        parts = interleaved_parts(len(rows), 64)
        rows_job = jobs.map(lambda p: rows_forward_dq(qr[p], kc, vc, dor[p], rows[p], causal=False,
                                                      doc_offsets=offsets), parts, "rows (O, LSE, dQ)")
        keys_job = jobs.map(doc_keys, short, "keys in the shortest documents")
        r = None
        for hc in w.head_chunks:
            print(f"   head_chunk={hc}", flush=True)
            cur = run(q, k, v, do, hc, causal=False, doc_offsets=offs_t)
            if r is None:
                r = cur
            else:
                for name in cur:
                    assert bit_equal(cur[name], r[name]), f"{name}: head_chunk {hc} differs"
                del cur
        gs = grad_scale(w)
        o_ref, l_ref, dq_ref = np.empty_like(qr), np.empty((w.Hq, len(rows))), np.empty_like(qr)
        for p, (o, lse, dq) in zip(parts, jobs.gather(rows_job)):
            o_ref[p], l_ref[:, p], dq_ref[p] = o, lse, dq
        assert_close("out", f64(r["out"][rows_t]), o_ref, w.dtype, per_item=True)
        assert_close("lse", f64(r["lse"][:, rows_t]), l_ref, w.dtype)
        assert_close("dq", f64(r["dq"][rows_t]), dq_ref, w.dtype, grad_scale=gs, per_item=True)
        for (start, end), (dk_ref, dv_ref) in zip(short, jobs.gather(keys_job)):
            keys_t = torch.arange(start, start + min(64, end - start), device=dev)
            assert_close("dk", f64(r["dk"][keys_t]), dk_ref, w.dtype, grad_scale=gs, per_item=True)
            assert_close("dv", f64(r["dv"][keys_t]), dv_ref, w.dtype, grad_scale=gs, per_item=True)
