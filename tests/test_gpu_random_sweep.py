"""A seeded random sweep of small problems: the HIP path through the C ABI
against the fp64 CPU oracle on full tensors.

Each case draws the sequence length (uniformly or on a 64/128/256 tile edge,
plus or minus one), one or two kv heads, 1 to 4 query heads per kv head, d of
64 or 128, bf16 or fp32, causal or not, and sometimes packed documents at
random offsets (empty and length-one documents possible). It runs head_chunk 1
and one other valid chunk size, compares out, lse, dq, dk and dv with the
oracle under the suite's tolerances, and requires the two chunk sizes to give
the same bits. Where the fused backward applies (bf16, d = 128, no documents)
it is checked the same way. The cases are fixed by one seed, so every run
checks the same problems; each prints its shape before it runs.
"""

import numpy as np
import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import assert_close, bit_equal, f64, grad_scale, run
from long_context_attention_upipe_amd.workloads import custom, make_inputs
from oracle.attention import attention_backward, attention_forward

pytestmark = pytest.mark.gpu


def _draw_cases(n=40, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "fp32" if rng.random() < 0.25 else "bf16"
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 3, 4]))
        Hq = Hkv * G
        s_max = 1200 if dtype == "fp32" else 2100
        if rng.random() < 0.5:
            S = int(rng.integers(1, s_max + 1))
        else:
            edge = int(rng.choice([64, 128, 256])) * int(rng.integers(1, s_max // 256 + 1))
            S = max(1, min(s_max, edge + int(rng.integers(-1, 2))))
        causal = bool(rng.random() < 0.75)
        docs = None
        if rng.random() < 0.35:
            cuts = sorted(int(x) for x in rng.integers(0, S + 1, size=int(rng.integers(1, 5))))
            docs = [0] + cuts + [S]
        valid = [hc for hc in range(2, Hq + 1) if Hq % hc == 0 and (G % hc == 0 or hc % G == 0)]
        hcs = (1, int(rng.choice(valid))) if valid else (1,)
        cases.append((S, Hq, Hkv, d, dtype, causal, docs, hcs, 7000 + i))
    return cases


CASES = _draw_cases()


def _id(c):
    S, Hq, Hkv, d, dtype, causal, docs, hcs, _ = c
    return (f"S{S}-h{Hq}x{Hkv}-d{d}-{dtype}-{'causal' if causal else 'full'}"
            f"{'-docs%d' % (len(docs) - 1) if docs else ''}-hc{'_'.join(map(str, hcs))}")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_problem_matches_oracle(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    S, Hq, Hkv, d, dtype, causal, docs, hcs, seed = case
    print(f"\n  sweep case {_id(case)} seed={seed}", flush=True)
    w = custom(S, Hq, Hkv, d, dtype, seed=seed, dout_scaled=dtype == "bf16", causal=causal)
    q, k, v, do = make_inputs(w, device="cpu")
    ro, rl = attention_forward(f64(q), f64(k), f64(v), causal=causal, doc_offsets=docs)
    rdq, rdk, rdv = attention_backward(f64(q), f64(k), f64(v), f64(do), causal=causal, doc_offsets=docs)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    offs = torch.tensor(docs, dtype=torch.int32, device=dev) if docs else None
    gs = grad_scale(w)
    fused_ok = dtype == "bf16" and d == 128 and docs is None

    def check(r):
        assert_close("dq", f64(r["dq"]), rdq, dtype, grad_scale=gs, per_item=True)
        assert_close("dk", f64(r["dk"]), rdk, dtype, grad_scale=gs, per_item=True)
        assert_close("dv", f64(r["dv"]), rdv, dtype, grad_scale=gs, per_item=True)

    first = first_fused = None
    for hc in hcs:
        print(f"   head_chunk={hc}", flush=True)
        r = run(qd, kd, vd, dod, hc, causal=causal, doc_offsets=offs)
        assert_close("out", f64(r["out"]), ro, dtype)
        assert_close("lse", f64(r["lse"]), rl, dtype)
        check(r)
        if first is None:
            first = r
        else:
            for name in r:
                assert bit_equal(r[name], first[name]), f"{name} differs between head_chunk {hcs[0]} and {hc}"
        if fused_ok:
            print(f"   fused backward, head_chunk={hc}", flush=True)
            out, lse, out_lo = up.attention_forward(qd, kd, vd, head_chunk=hc, causal=causal)
            dq, dk, dv = up.attention_backward_fused(qd, kd, vd, out, dod, lse, out_lo, head_chunk=hc, causal=causal)
            torch.cuda.synchronize()
            rf = dict(dq=dq, dk=dk, dv=dv)
            check(rf)
            if first_fused is None:
                first_fused = rf
            else:
                for name in rf:
                    assert bit_equal(rf[name], first_fused[name]), f"fused {name} differs across head_chunk"
