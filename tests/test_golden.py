"""Regression fixture: the oracle still reproduces the values it froze.

The pages print no worked example, so the fixture holds the oracle's own
outputs (written by tests/golden/make_golden.py, which calls only oracle/).
The row-0 entries also have a closed form, checked here independently.
"""

import json
import math
import os

import numpy as np

from oracle.attention import attention_backward, attention_forward

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "small_causal_gqa.json")


def test_oracle_reproduces_frozen_fixture():
    with open(GOLDEN) as f:
        g = json.load(f)
    q, k, v, do = (np.array(g[n]) for n in ("q", "k", "v", "dout"))
    out, lse = attention_forward(q, k, v, causal=True)
    dq, dk, dv = attention_backward(q, k, v, do, causal=True)
    for name, val in (("out", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(val, np.array(g[name]), rtol=1e-13, atol=1e-14, err_msg=name)
    # closed form for causal row 0: O_0 = v_0, LSE_0 = <q_0,k_0>/sqrt(d)
    d = q.shape[2]
    for h in range(q.shape[1]):
        assert np.array(g["out"])[0, h].tolist() == v[0, 0].tolist()
        assert math.isclose(g["lse"][h][0], float(q[0, h] @ k[0, 0]) / math.sqrt(d), rel_tol=1e-14)
