"""The cross-entropy oracle against its pins, and planted mistakes that some
pin must catch (CPU only)."""

import os
import types

import pytest

import oracle.loss as lmod
from oracle_pins import CE_PINS, failing_ce_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "loss.py")


@pytest.mark.parametrize("pin", CE_PINS, ids=lambda p: p.__name__)
def test_ce_pin(pin):
    pin(lmod)


MUTATIONS = {
    "log2": ("lse = (m + np.log(np.exp(z - m)", "lse = (m + np.log2(np.exp(z - m)"),
    "missing_onehot": ("g[rows[counted], lab[counted]] -= 1.0", "pass"),
    "ignored_rows_kept": ("g[~counted] = 0.0", "pass"),
    "dh_transposed_w": ("dh[r0:r1] = g @ w", "dh[r0:r1] = (g @ w)[::-1]"),
    "dw_missing_scale": ("g *= scale", "g *= 1.0"),
    "loss_sign": ("loss[r0:r1] = np.where(counted, lse - picked, 0.0)", "loss[r0:r1] = np.where(counted, picked - lse, 0.0)"),
    "dw_last_block_only": ("dw += g.T @ h[r0:r1]", "dw = g.T @ h[r0:r1]"),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("loss_mutant")
    exec(compile(src.replace(old, new, 1), "loss_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_loss_mistake_is_caught(name):
    assert failing_ce_pins(_mutant(*MUTATIONS[name])), f"no pin catches {name}"
