"""The SwiGLU MLP oracle against its pins, and planted mistakes that some pin
must catch (CPU only)."""

import os
import types

import pytest

import oracle.mlp as mmod
from oracle_pins import MLP_PINS, failing_mlp_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "mlp.py")


@pytest.mark.parametrize("pin", MLP_PINS, ids=lambda p: p.__name__)
def test_mlp_pin(pin):
    pin(mmod)


MUTATIONS = {
    "silu_without_z": ("a = round_bf16(g * sg * u)", "a = round_bf16(sg * u)"),
    "gate_up_swapped": ("a = round_bf16(g * sg * u)", "a = round_bf16(u * _sigmoid(u) * g)"),
    "dsilu_missing_term": ("dg = da * u * sg * (1.0 + g * (1.0 - sg))", "dg = da * u * sg"),
    "da_transposed": ("da = dy @ wd", "da = (dy @ wd)[:, ::-1]"),
    "dwd_uses_g": ("dy.T @ a)", "dy.T @ g)"),
    "dx_missing_up": ("dx = dg @ wg + du @ wu", "dx = dg @ wg"),
    "y_not_rounded": ("y = round_bf16(a @ wd.T)", "y = a @ wd.T"),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1).replace("from .block import", "from oracle.block import")
    mod = types.ModuleType("mlp_mutant")
    exec(compile(src, "mlp_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mlp_mistake_is_caught(name):
    assert failing_mlp_pins(_mutant(*MUTATIONS[name])), f"no pin catches {name}"
