"""A seeded random sweep of the attention block (per-chunk q/k/v projections,
attention, output projection; forward and backward) through the C ABI
against the oracle on full tensors.

Each case draws S, the model dim Dm (a multiple of 64), one or two kv heads,
1, 2 or 4 query heads per kv head, d of 64 or 128 and causal or not, and runs
head_chunk 1 and one other valid chunk size: y, out and lse of the forward,
and dx and the four weight gradients of the backward with o recomputed, must
match the oracle under the fixed-shape tests' bounds and be bit-identical
across the two chunk sizes. The cases are fixed by one seed; each prints its
shape first.
"""

import numpy as np
import pytest

from gpu_util import assert_close, bit_equal, f64
from long_context_attention_upipe_amd.workloads import make_block_inputs
from oracle.block import attention_block_backward, attention_block_forward
from test_gpu_block import GRADS, _bf16, _block_bwd_run, _block_run, _check_grads, _dev

pytestmark = pytest.mark.gpu


def _draw_cases(n=10, seed=8080):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        S = int(rng.integers(1, 2500))
        Dm = 64 * int(rng.integers(1, 9))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4]))
        Hq = Hkv * G
        d = int(rng.choice([64, 128]))
        causal = bool(rng.random() < 0.75)
        valid = [hc for hc in range(2, Hq + 1) if Hq % hc == 0 and (G % hc == 0 or hc % G == 0)]
        hcs = (1, int(rng.choice(valid))) if valid else (1,)
        cases.append((S, Dm, Hq, Hkv, d, causal, hcs, 1100 + i))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("case", CASES, ids=["S%d-Dm%d-h%dx%d-d%d-%s-hc%s" % (c[0], c[1], c[2], c[3], c[4],
                                                                             "causal" if c[5] else "full",
                                                                             "_".join(map(str, c[6])))
                                             for c in CASES])
def test_random_block_matches_oracle(case):
    dev = _dev()
    S, Dm, Hq, Hkv, d, causal, hcs, seed = case
    print(f"\n  block case S={S} Dm={Dm} Hq={Hq} Hkv={Hkv} d={d} causal={causal} head_chunks={hcs}", flush=True)
    x, wq, wk, wv, wo = make_block_inputs(S, Dm, Hq, Hkv, d, seed=seed, device=dev)
    dy = _bf16((S, Dm), seed + 1, dev)
    y_ref, o_ref, l_ref = attention_block_forward(*(f64(t) for t in (x, wq, wk, wv, wo)), Hq, Hkv, causal=causal)
    refs = attention_block_backward(*(f64(t) for t in (x, wq, wk, wv, wo, dy)), Hq, Hkv, causal=causal)
    first_f = first_b = None
    for hc in hcs:
        print(f"   head_chunk={hc}", flush=True)
        f = _block_run(x, wq, wk, wv, wo, Hq, Hkv, hc, causal)
        assert_close("y", f64(f[0]), y_ref, "bf16", per_item=True)
        assert_close("out", f64(f[1]), o_ref, "bf16", per_item=True)
        assert_close("lse", f64(f[2]), l_ref, "bf16")
        b = _block_bwd_run(x, wq, wk, wv, wo, dy, Hq, Hkv, hc, causal)
        _check_grads(b, refs)
        if first_f is None:
            first_f, first_b = f, b
        else:
            for name, u, w in zip(("y", "out", "lse"), f, first_f):
                assert bit_equal(u, w), f"{name} differs between head_chunk {hcs[0]} and {hc}"
            for name, u, w in zip(GRADS, b, first_b):
                assert bit_equal(u, w), f"{name} differs between head_chunk {hcs[0]} and {hc}"
