"""The block oracle (projections + attention) against its pins, and planted
mistakes that some pin must catch (CPU only)."""

import os
import types

import pytest

import oracle.attention as amod
import oracle.block as bmod
from oracle_pins import BLOCK_PINS, failing_block_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "block.py")


@pytest.mark.parametrize("pin", BLOCK_PINS, ids=lambda p: p.__name__)
def test_block_pin(pin):
    pin(bmod, amod)


MUTATIONS = {
    "q_not_transposed": ("q = rnd(x @ wq.T)", "q = rnd((wq @ x.T).T[:, ::-1])"),
    "heads_d_major": ("q = rnd(x @ wq.T).reshape(S, n_q_heads, d)",
                      "q = rnd(x @ wq.T).reshape(S, d, n_q_heads).transpose(0, 2, 1)"),
    "q_not_rounded": ("q = rnd(x @ wq.T)", "q = (x @ wq.T)"),
    "o_not_rounded": ("o = rnd(out)", "o = out"),
    "k_from_wv": ("k = rnd(x @ wk.T)", "k = rnd(x @ wv.T)"),
    "wo_columns": ("y = o.reshape(S, n_q_heads * d) @ wo.T", "y = o.reshape(S, n_q_heads * d) @ wo[:, ::-1].T"),
    "round_truncates": ("bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16 << 16", "bits = bits >> 16 << 16"),
    "round_ties_up": ("bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16 << 16", "bits = (bits + 0x8000) >> 16 << 16"),
    "rows_q_all_rows": ("q = round_bf16(x[rows] @ wq.T)", "q = round_bf16(x[rows[::-1]] @ wq.T)"),
    "rows_v_from_wk": ("v = round_bf16(x @ wv.T).reshape(S, n_kv_heads, d)\n    q = round_bf16",
                       "v = round_bf16(x @ wk.T).reshape(S, n_kv_heads, d)\n    q = round_bf16"),
    "non_causal": ("out, lse = attention_forward(q, k, v, causal=causal)",
                   "out, lse = attention_forward(q, k, v, causal=False)"),
    "bwd_o_not_rounded": ("o = rnd(out).reshape(S, n_q_heads * d)", "o = out.reshape(S, n_q_heads * d)"),
    "bwd_do_columns": ("do = (dy @ wo)", "do = (dy @ wo[:, ::-1])"),
    "bwd_dwo_from_do": ("dwo = dy.T @ o", "dwo = dy.T @ (dy @ wo)"),
    "bwd_dx_missing_dv": ("dx = dq @ wq + dk @ wk + dv @ wv", "dx = dq @ wq + dk @ wk"),
    "bwd_dx_dk_through_wv": ("dx = dq @ wq + dk @ wk + dv @ wv", "dx = dq @ wq + dk @ wv + dv @ wv"),
    "bwd_non_causal": ("dq, dk, dv = attention_backward(q, k, v, do, causal=causal)",
                       "dq, dk, dv = attention_backward(q, k, v, do, causal=False)"),
    "bwd_dwk_dwv_swapped": ("dq.T @ x, dk.T @ x, dv.T @ x", "dq.T @ x, dv.T @ x, dk.T @ x"),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("block_mutant")
    exec(compile(src, "block_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_block_mistake_is_caught(name):
    assert failing_block_pins(_mutant(*MUTATIONS[name]), amod), f"no pin catches {name}"


def test_unmutated_block_copy_passes():
    with open(SRC) as f:
        src = f.read().replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("block_copy")
    exec(compile(src, "block_copy.py", "exec"), mod.__dict__)
    assert failing_block_pins(mod, amod) == []
