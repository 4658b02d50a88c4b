"""Write tests/golden/small_causal_gqa.json from the CPU oracle alone.

The pages print no worked numerical example for attention (the talk digest
says the talk gives no figures, code or configs), so the only stored values
here are the oracle's own, frozen as a regression fixture. The inputs are
small exact dyadic numbers so that the fixture is exact to read back.

Run:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.attention import attention_backward, attention_forward  # noqa: E402


def inputs():
    S, Hq, Hkv, d = 5, 2, 1, 4
    # quarters in [-2, 2): exact in bf16, fp32 and fp64
    rng = np.random.default_rng(20261202)
    q = rng.integers(-8, 8, size=(S, Hq, d)) / 4.0
    k = rng.integers(-8, 8, size=(S, Hkv, d)) / 4.0
    v = rng.integers(-8, 8, size=(S, Hkv, d)) / 4.0
    do = rng.integers(-8, 8, size=(S, Hq, d)) / 4.0
    return q, k, v, do


def main():
    q, k, v, do = inputs()
    out, lse = attention_forward(q, k, v, causal=True)
    dq, dk, dv = attention_backward(q, k, v, do, causal=True)
    doc = {
        "what": "causal GQA attention, S=5, Hq=2, Hkv=1, d=4, tau=1/sqrt(d); oracle outputs frozen",
        "written_by": "tests/golden/make_golden.py (calls only oracle/)",
        "layout": "q,k,v,dout,out,dq,dk,dv are [S,H,d]; lse is [Hq,S] natural log",
        "q": q.tolist(), "k": k.tolist(), "v": v.tolist(), "dout": do.tolist(),
        "out": out.tolist(), "lse": lse.tolist(), "dq": dq.tolist(), "dk": dk.tolist(), "dv": dv.tolist(),
    }
    with open(os.path.join(HERE, "small_causal_gqa.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
