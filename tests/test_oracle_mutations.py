"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
at least one pin catches each: the pins are strong enough to trust."""

import importlib.util
import os
import types

import pytest

from oracle_pins import failing_pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTATIONS = {
    "scale_1_over_d": ("tau = 1.0 / math.sqrt(d)", "tau = 1.0 / d"),
    "diagonal_excluded": ("np.arange(n_cols)[None, :] > rows[:, None]", "np.arange(n_cols)[None, :] >= rows[:, None]"),
    "gqa_modulo_mapping": ("return h // (n_q_heads // n_kv_heads)", "return h % n_kv_heads"),
    "lse_base2": ("return e / l, (m + np.log(l))[..., 0]", "return e / l, (m + np.log2(l))[..., 0]"),
    "lse_missing_max": ("return e / l, (m + np.log(l))[..., 0]", "return e / l, (np.log(l))[..., 0]"),
    "bwd_missing_D": ("ds = p * (dp - D[:, None])", "ds = p * dp"),
    "bwd_dk_missing_tau": ("dk[:n_cols, g, :] += tau * (ds.T @ q_blk)", "dk[:n_cols, g, :] += (ds.T @ q_blk)"),
    "bwd_dv_uses_ds": ("dv[:n_cols, g, :] += p.T @ do_blk", "dv[:n_cols, g, :] += ds.T @ do_blk"),
    "bwd_dq_transposed_k": ("dq[r0:r1, h, :] = tau * (ds @ k[:n_cols, g, :])", "dq[r0:r1, h, :] = tau * (ds @ v[:n_cols, g, :])"),
    "cols_wrong_causal_side": ("(need[None, :] < cj[:, None])", "(need[None, :] > cj[:, None])"),
    "cols_dv_missing": ("dv[c0:c0 + per, g, :] += p @ doh", "dv[c0:c0 + per, g, :] += 0 * (p @ doh)"),
    "fwd_rows_noncausal_width": ("        n_cols = int(r.max()) + 1 if causal else S\n        mask = _look_back_mask(r, n_cols, causal, bounds)\n        for g in range(Hkv):\n            hs = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]\n            s = _group_scores(q_rows[sel][:, hs, :], k[:n_cols, g, :], tau, mask)\n            p, lse_blk",
                                 "        n_cols = int(r.max()) + 1\n        mask = _look_back_mask(r, n_cols, causal, bounds)\n        for g in range(Hkv):\n            hs = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]\n            s = _group_scores(q_rows[sel][:, hs, :], k[:n_cols, g, :], tau, mask)\n            p, lse_blk"),
    "rows_dq_missing_D": ("            ds = p * (dp - D[..., None])", "            ds = p * dp"),
    "group_scores_mask_ignored": ("        s[np.broadcast_to(mask[:, None, :], s.shape)] = -np.inf", "        pass"),
    "softmax_wrong_axis": ("    m = s.max(axis=-1, keepdims=True)", "    m = s.max(axis=0, keepdims=True)"),
    "docs_last_off_by_one": ("return off[doc], off[doc + 1] - 1", "return off[doc], off[doc + 1]"),
    "docs_search_left": ('doc = np.searchsorted(off, np.arange(S), side="right") - 1',
                         'doc = np.searchsorted(off, np.arange(S), side="left") - 1'),
    "docs_mask_no_lower": ("outside = (cols < first[rows][:, None]) | (cols > last[rows][:, None])",
                           "outside = (cols > last[rows][:, None])"),
    "docs_mask_no_upper": ("outside = (cols < first[rows][:, None]) | (cols > last[rows][:, None])",
                           "outside = (cols < first[rows][:, None])"),
    "docs_mask_replaces_causal": ("mask = outside if mask is None else (mask | outside)", "mask = outside"),
    "cols_docs_ignored": ("excluded = other_doc if excluded is None else (excluded | other_doc)", "pass"),
    "cols_docs_first_row": ("first = max(first, int(bounds[0][cols].min()))", "first = max(first, int(bounds[0][cols].max()))"),
    "fused_rows_missing_D": ("            ds = p * (_rows_matmul(do_blk, v_g.T) - D[..., None])",
                             "            ds = p * _rows_matmul(do_blk, v_g.T)"),
    "fused_rows_dq_uses_v": ("            dq[np.ix_(sel, hs)] = tau * _rows_matmul(ds, k_g)",
                             "            dq[np.ix_(sel, hs)] = tau * _rows_matmul(ds, v_g)"),
    "fused_rows_dq_missing_tau": ("            dq[np.ix_(sel, hs)] = tau * _rows_matmul(ds, k_g)",
                                  "            dq[np.ix_(sel, hs)] = _rows_matmul(ds, k_g)"),
    "fused_rows_D_from_v": ("            D = (do_blk * o).sum(axis=-1)\n            ds = p * (_rows_matmul(do_blk, v_g.T)",
                            "            D = (do_blk * v_g[:1]).sum(axis=-1)\n            ds = p * (_rows_matmul(do_blk, v_g.T)"),
    "fused_rows_lse_transposed_heads": ("            lse[np.ix_(hs, sel)] = lse_blk.T\n            do_blk",
                                        "            lse[np.ix_(hs, sel)] = lse_blk.T[::-1]\n            do_blk"),
    "cols_row_stats_swapped": ("        o_need, lse_need = _f64(row_stats[0]), _f64(row_stats[1])",
                               "        o_need, lse_need = _f64(row_stats[0]), _f64(row_stats[1])[::-1]"),
    "cols_docs_end_row": ("end = int(bounds[1][cols].max()) + 1", "end = int(bounds[1][cols].min()) + 1"),
}


def _mutant(old, new):
    with open(SRC_PATH) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    bad = failing_pins(_mutant(old, new))
    assert bad, f"no pin catches the planted mistake {name}"


def test_unmutated_copy_passes_every_pin():
    with open(SRC_PATH) as f:
        src = f.read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy.py", "exec"), mod.__dict__)
    assert failing_pins(mod) == []
