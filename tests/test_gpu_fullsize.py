"""Full-size workloads through the C ABI, checked against the oracle.

From S = 131,072 up, checks on seeded samples:
  * O, LSE and dQ at 4096 seeded sampled query rows (first/last rows, both
    sides of tile boundaries, the rest uniform) are exact in O(S*d) per row
    (one score pass per row gives all three);
  * dK and dV at seeded keys in the last positions are exact too, since only
    the rows after them contribute;
  * sum_j dK_j = 0 and sum_j dV_j = sum of dO over the group hold at any size;
  * outputs are bit-identical across every head_chunk tested.
At 131,072 tokens the same workload is also checked on the full tensors,
every dK/dV key tile included.
The launch configuration is the one bench.py times (same workload table,
same inputs, same entry points). The oracle runs on host threads while the
GPU computes; gradients are compared at unit dO scale, and every sampled row
and key is bounded on its own as well as the tensor as a whole.
"""

import numpy as np
import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import TOL, OracleJobs, assert_close, bit_equal, f64, grad_scale, interleaved_parts, progress, sum64
from long_context_attention_upipe_amd.workloads import WORKLOADS, Workload, make_inputs, sample_rows, tail_keys
from oracle.attention import backward_cols_dkdv, cols_rows_needed, forward_rows, rows_forward_dq

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _run_chunks(w, q, k, v, do, head_chunks, causal=True, fused=False):
    """Forward + backward (the two-kernel one, or the fused one) at every
    head_chunk; returns the first one's outputs after checking that the others
    are bit-identical to it."""
    results = {}
    for hc in head_chunks:
        progress(f"   {w.name}: head_chunk={hc} causal={causal} fused={fused}")
        ws = up.workspace(w.S, w.Hq, w.Hkv, w.d, hc, q.dtype, q.device, "fwd" if fused else "both")
        up.upipe_profile_reset()
        up.upipe_profile_enable(True)
        out, lse, out_lo = up.attention_forward(q, k, v, head_chunk=hc, causal=causal, ws=ws)
        if fused:
            del ws
            dq, dk, dv = up.attention_backward_fused(q, k, v, out, do, lse, out_lo, head_chunk=hc, causal=causal)
            ws = None
        else:
            dq, dk, dv = up.attention_backward(q, k, v, out, do, lse, out_lo, head_chunk=hc, causal=causal, ws=ws)
        up.wait_reporting(f"head_chunk={hc}", q.device, prefix="  ", log=progress)
        up.upipe_profile_enable(False)
        up.upipe_profile_reset()
        del ws, out_lo
        results[hc] = dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv)
        if len(results) > 1:
            first = results[head_chunks[0]]
            for name in results[hc]:
                assert bit_equal(results[hc][name], first[name]), f"{name}: head_chunk {hc} differs"
            del results[hc]
    return results[head_chunks[0]]


def _check(w, head_chunks, n_rows, n_keys, key_window, causal=True, fused=False):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    progress(f"\n  case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} head_chunks={head_chunks} causal={causal} "
             f"rows={n_rows} keys={n_keys if causal else 0} fused={fused}")
    dev = torch.device("cuda:0")
    q, k, v, do = make_inputs(w, device=dev)
    rows = sample_rows(w.S, n_rows, seed=w.seed + 7)
    rows_t = torch.from_numpy(rows).to(dev)
    kc, vc = f64(k), f64(v)
    qr, dor = f64(q[rows_t]), f64(do[rows_t])
    with OracleJobs() as jobs:
        # host side, concurrent with the GPU run below
        parts = interleaved_parts(len(rows), 64)
        rows_job = jobs.map(lambda p: rows_forward_dq(qr[p], kc, vc, dor[p], rows[p], causal=causal), parts,
                            "rows (O, LSE, dQ)")
        stats_job = None
        if causal:
            keys = tail_keys(w.S, n_keys, key_window, seed=w.seed + 8)
            # The keys' gradients need the softmax rows (O, LSE) of every row
            # after the first key: that forward runs in pieces on the pool.
            need = cols_rows_needed(keys, w.S)
            qn = f64(q[torch.from_numpy(need).to(dev)])
            stat_parts = interleaved_parts(len(need), 16)
            stats_job = jobs.map(lambda p: forward_rows(qn[p], kc, vc, need[p]), stat_parts,
                                 "rows the tail keys need (O, LSE)")
            # Only rows at or after the first sampled key contribute to it; the
            # rest of these float32 arrays stays as untouched zero pages.
            # float32 holds bf16 values exactly; the oracle upcasts what it reads.
            first = int(need[0])
            q32 = np.zeros(tuple(q.shape), dtype=np.float32)
            do32 = np.zeros(tuple(do.shape), dtype=np.float32)
            q32[first:], do32[first:] = q[first:].float().cpu().numpy(), do[first:].float().cpu().numpy()

        r = _run_chunks(w, q, k, v, do, head_chunks, causal, fused)

        gs = grad_scale(w)
        o_ref, l_ref, dq_ref = np.empty_like(qr), np.empty((w.Hq, len(rows))), np.empty_like(qr)
        for p, (o, lse, dq) in zip(parts, jobs.gather(rows_job)):
            o_ref[p], l_ref[:, p], dq_ref[p] = o, lse, dq
        assert_close("out", f64(r["out"][rows_t]), o_ref, w.dtype, per_item=True)
        assert_close("lse", f64(r["lse"][:, rows_t]), l_ref, w.dtype)
        assert_close("dq", f64(r["dq"][rows_t]), dq_ref, w.dtype, grad_scale=gs, per_item=True)
        if stats_job is not None:
            o_need, l_need = np.empty((len(need), w.Hq, w.d)), np.empty((w.Hq, len(need)))
            for p, (o, lse) in zip(stat_parts, jobs.gather(stats_job)):
                o_need[p], l_need[:, p] = o, lse
            dk_ref, dv_ref = backward_cols_dkdv(q32, kc, vc, do32, keys, row_stats=(o_need, l_need))
            keys_t = torch.from_numpy(keys).to(dev)
            assert_close("dk", f64(r["dk"][keys_t]), dk_ref, w.dtype, grad_scale=gs, per_item=True)
            assert_close("dv", f64(r["dv"][keys_t]), dv_ref, w.dtype, grad_scale=gs, per_item=True)

    print("   identities: column sums", flush=True)
    G = w.Hq // w.Hkv
    dk_sum, dk_abs = sum64(r["dk"], (0,)), sum64(r["dk"].abs(), (0,))
    dv_sum = sum64(r["dv"], (0,))
    for g in range(w.Hkv):
        assert np.all(np.abs(dk_sum[g]) <= 1e-2 * dk_abs[g] + 1e-4)
        ref = sum64(do[:, g * G:(g + 1) * G, :], (0, 1))
        assert_close("dvsum", dv_sum[g], ref, w.dtype)
    return r


def test_llama8b_share_128k_sampled_4096_rows():
    w = WORKLOADS["llama8b_share_s128k"]
    _check(w, w.head_chunks, 4096, 256, 2048)


def test_llama8b_share_1m_sampled_4096_rows():
    w = WORKLOADS["llama8b_share_s1m"]
    _check(w, w.head_chunks, 4096, 128, 512)


def test_llama8b_share_3m_sampled_4096_rows():
    """3,145,728 tokens (the length the talk's technique stack reaches without
    UPipe), every head_chunk of the workload, bit-identical across them."""
    w = WORKLOADS["llama8b_share_s3m"]
    _check(w, w.head_chunks, 4096, 64, 256)


def test_share32b_5m_sampled_4096_rows():
    """5,242,880 tokens, Hq = 8 (the 32B share the talk reaches with UPipe),
    at head_chunk 1: the smallest pool, the configuration the method exists
    for. Larger head_chunks run the same kernels in wider launches; their bit
    identity with head_chunk 1 is checked at 128K, 1M and 3M tokens."""
    w = WORKLOADS["share32b_s5m"]
    _check(w, (1,), 4096, 64, 128)


def test_head_dim_64_two_kv_heads_ragged_131k_sampled_rows():
    """Head dim 64 (its own kernel instantiations and LDS layouts), two kv
    heads (Hq = 8, Hkv = 2) and a length that is no multiple of any tile
    (131,109 = 2^17 + 37), at head_chunk 1, 2, 4 (chunks inside one kv group)
    and 8 (both groups in one chunk): the same sampled-row, tail-key and
    column-sum checks as the workloads above, and bit-identity across
    head_chunk."""
    w = Workload("d64_gqa2_s131109", 131109, 8, 2, 64, "bf16", (1, 2, 4, 8), True, 7000)
    _check(w, w.head_chunks, 2048, 128, 1024)


def test_llama8b_share_128k_non_causal_sampled_rows():
    """Non-causal attention (every row sees all S keys) at 131,072 tokens: O,
    LSE and dQ at 2048 sampled rows, exact in O(S*d) each; bit-identity across
    head_chunk; the column sums sum_j dK_j = 0 and sum_j dV_j = sum of dO over
    the group, which hold without a mask too. Sampled dK/dV keys are not
    checked here: without the causal mask every row contributes to every key,
    so exact values need every row's LSE and D, O(S^2 d)."""
    w = WORKLOADS["llama8b_share_s128k"]
    _check(w, w.head_chunks, 2048, 0, 0, causal=False)


def test_llama8b_share_128k_full_tensors_every_head_chunk():
    """The 131,072-token workload (the 8B share: Hq = 4, Hkv = 1, d = 128,
    bf16, dO ~ N(0,1)/sqrt(S)), every element of out, lse, dq, dk and dv
    against the oracle, at head_chunk 1, 2 and 4 (bit-identical). The dK/dV
    grid has 1024 key tiles here, so its XCD-aware tile order (runs of 8 tiles
    per block of 64 workgroups) is covered element by element, heavy early
    key tiles included. The full-tensor reference is assembled from the
    oracle's per-row function over every row (O, LSE, dQ) and its per-key
    function over every key (dK, dV, from those rows' O and LSE), both pinned
    equal to the full-tensor functions, so that it runs in parts on
    single-threaded BLAS."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = WORKLOADS["llama8b_share_s128k"]
    progress(f"\n  case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} head_chunks={w.head_chunks} full tensors")
    dev = torch.device("cuda:0")
    q, k, v, do = make_inputs(w, device=dev)
    qc, kc, vc, doc = f64(q), f64(k), f64(v), f64(do)
    rows = np.arange(w.S)
    with OracleJobs() as jobs:
        parts = interleaved_parts(w.S, 256)
        rows_job = jobs.map(lambda p: rows_forward_dq(qc[p], kc, vc, doc[p], rows[p]), parts,
                            "every row (O, LSE, dQ)")
        r = _run_chunks(w, q, k, v, do, w.head_chunks)
        o_ref, l_ref, dq_ref = np.empty_like(qc), np.empty((w.Hq, w.S)), np.empty_like(qc)
        for p, (o, lse, dq) in zip(parts, jobs.gather(rows_job)):
            o_ref[p], l_ref[:, p], dq_ref[p] = o, lse, dq
        # every key, in blocks; a block's keys need the rows from its first key on
        blocks = [(a, min(w.S, a + 2048)) for a in range(0, w.S, 2048)]
        cols_job = jobs.map(lambda ab: backward_cols_dkdv(qc, kc, vc, doc, np.arange(ab[0], ab[1]),
                                                          row_stats=(o_ref[ab[0]:], l_ref[:, ab[0]:])),
                            blocks, "every key (dK, dV)")
        dk_ref, dv_ref = np.empty_like(kc), np.empty_like(vc)
        for (a, b), (dk_b, dv_b) in zip(blocks, jobs.gather(cols_job)):
            dk_ref[a:b], dv_ref[a:b] = dk_b, dv_b
    gs = grad_scale(w)
    assert_close("out", f64(r["out"]), o_ref, w.dtype, per_item=True)
    assert_close("lse", f64(r["lse"]), l_ref, w.dtype)
    assert_close("dq", f64(r["dq"]), dq_ref, w.dtype, grad_scale=gs, per_item=True)
    assert_close("dk", f64(r["dk"]), dk_ref, w.dtype, grad_scale=gs, per_item=True)
    assert_close("dv", f64(r["dv"]), dv_ref, w.dtype, grad_scale=gs, per_item=True)


def test_llama8b_share_1m_fused_backward_sampled_4096_rows():
    """The fused deterministic backward at the bench workload (1,048,576
    tokens, head_chunk 1 and 4): sampled dQ rows and tail keys against the
    oracle, bit-identical across head_chunk, and every element within the
    bf16 tolerance of the two-kernel backward's."""
    w = WORKLOADS["llama8b_share_s1m"]
    r = _check(w, (1, 4), 4096, 128, 512, fused=True)
    progress("   every element against the two-kernel backward")
    q, k, v, do = make_inputs(w, device=torch.device("cuda:0"))
    ref = _run_chunks(w, q, k, v, do, (1,))
    gs = grad_scale(w)
    max_abs_tol, rel_tol = TOL[w.dtype]
    for name in ("dq", "dk", "dv"):
        # on the device, in float32 (both sides are bf16): the same bounds as
        # against the oracle, at unit dO scale
        a, b = r[name].float() * gs, ref[name].float() * gs
        err = (a - b).abs()
        worst = float((err / b.abs().clamp_min(1.0)).max())
        rel = float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))
        progress(f"   {name}: max |err| / max(|ref|, 1) = {worst:.3e}, relative Frobenius {rel:.3e}")
        assert torch.isfinite(a).all()
        assert worst <= max_abs_tol and rel <= rel_tol, name
