"""The CPU oracle against its pins (library routines, finite differences,
closed forms and identities) -- no GPU needed."""

import numpy as np
import pytest

import oracle.attention as oracle_mod
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_mod)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,Hq,Hkv,d", [(1, 1, 1, 1), (2, 1, 1, 4), (3, 4, 1, 4), (17, 4, 2, 64), (64, 2, 2, 4), (130, 4, 1, 8)])
def test_oracle_vs_sdpa_shapes(S, Hq, Hkv, d, causal):
    from oracle_pins import pin_sdpa_forward
    pin_sdpa_forward(oracle_mod, S=S, Hq=Hq, Hkv=Hkv, d=d, causal=causal)


@pytest.mark.parametrize("causal", [True, False])
def test_oracle_backward_vs_autograd_noncausal_and_mha(causal):
    from oracle_pins import pin_sdpa_backward
    pin_sdpa_backward(oracle_mod, S=19, Hq=3, Hkv=3, d=4, causal=causal)


def test_finite_differences_noncausal():
    from oracle_pins import pin_finite_differences
    pin_finite_differences(oracle_mod, causal=False)


def test_block_size_does_not_matter():
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((40, 2, 8)), rng.standard_normal((40, 1, 8)), rng.standard_normal((40, 1, 8))
    a = oracle_mod.attention_forward(q, k, v, block=1)
    b = oracle_mod.attention_forward(q, k, v, block=40)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13, atol=1e-14)


def test_kv_head_mapping_rejects_bad_groups():
    with pytest.raises(ValueError):
        oracle_mod.kv_head_of(0, 4, 3)
    assert [oracle_mod.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
