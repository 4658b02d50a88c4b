"""Seeded random sweeps of the sequence-tiled loss and MLP through the C ABI
against the oracle.

Loss cases draw S, Dm (a multiple of 64), V (a multiple of 8), the tile (a
multiple of 64, from smaller than S to larger) and a share of ignored labels;
MLP cases draw S, Dm, F (multiples of 64) and the tile. Both check every
output and gradient under the bounds of the fixed-shape tests, and a repeated
call must give the same bits. The cases are fixed by one seed; each prints
its shape first.
"""

import numpy as np
import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import assert_close, bit_equal, f64
from oracle.loss import cross_entropy
from oracle.mlp import swiglu_mlp

pytestmark = pytest.mark.gpu


def _loss_cases(n=12, seed=515):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(rng.integers(1, 3000))
        Dm = 64 * int(rng.integers(1, 9))
        V = 8 * int(rng.integers(1, 750))
        tile = 64 * int(rng.integers(1, 17))
        ignore = float(rng.choice([0.0, 0.0, 0.1, 0.5]))
        out.append((S, Dm, V, tile, ignore, 600 + i))
    return out


def _mlp_cases(n=12, seed=616):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        S = int(rng.integers(1, 3000))
        Dm = 64 * int(rng.integers(1, 9))
        F = 64 * int(rng.integers(1, 25))
        tile = 64 * int(rng.integers(1, 17))
        out.append((S, Dm, F, tile, 700 + i))
    return out


LOSS_CASES, MLP_CASES = _loss_cases(), _mlp_cases()


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _gen(seed):
    return torch.Generator(device="cpu").manual_seed(seed)


@pytest.mark.parametrize("case", LOSS_CASES, ids=["S%d-Dm%d-V%d-t%d-ign%g" % c[:5] for c in LOSS_CASES])
def test_random_tiled_loss_matches_oracle(case):
    dev = _dev()
    S, Dm, V, tile, ignore, seed = case
    print(f"\n  loss case S={S} Dm={Dm} V={V} tile={tile} ignored={ignore}", flush=True)
    g = _gen(seed)
    h = torch.randn((S, Dm), generator=g).to(torch.bfloat16)
    w = (torch.randn((V, Dm), generator=g) / Dm ** 0.5 * 2).to(torch.bfloat16)
    labels = torch.randint(0, V, (S,), generator=g, dtype=torch.int32)
    labels[torch.rand(S, generator=g) < ignore] = -100
    n = int((labels >= 0).sum())
    scale = 1.0 / max(1, n)
    h, w, labels = h.to(dev), w.to(dev), labels.to(dev)

    def call():
        ws = torch.empty(up.upipe_ce_loss_workspace_bytes(S, Dm, V, tile, True), dtype=torch.uint8, device=dev)
        loss = torch.full((S,), float("nan"), device=dev)
        dh = torch.full_like(h, float("nan"))
        dw = torch.full((V, Dm), float("nan"), device=dev)
        up.upipe_ce_loss_tiled(h, w, labels, loss, dh, dw, tile, scale, ws)
        torch.cuda.synchronize()
        return loss, dh, dw

    loss, dh, dw = call()
    rl, rdh, rdw = cross_entropy(f64(h), f64(w), labels.cpu().numpy(), scale=scale)
    assert_close("loss", f64(loss), rl, "bf16", per_item=False)
    if n:
        assert_close("dh", f64(dh), rdh, "bf16", grad_scale=float(n), per_item=True)
        assert_close("dw", f64(dw), rdw, "bf16", grad_scale=float(n), per_item=True, elem_floor="row")
    else:  # every label ignored: nothing to learn from
        assert float(dh.float().abs().max()) == 0.0 and float(dw.abs().max()) == 0.0
    for a, b in zip((loss, dh, dw), call()):
        assert bit_equal(a, b), "repeated call differs"


@pytest.mark.parametrize("case", MLP_CASES, ids=["S%d-Dm%d-F%d-t%d" % c[:4] for c in MLP_CASES])
def test_random_tiled_mlp_matches_oracle(case):
    dev = _dev()
    S, Dm, F, tile, seed = case
    print(f"\n  mlp case S={S} Dm={Dm} F={F} tile={tile}", flush=True)
    g = _gen(seed)
    x = torch.randn((S, Dm), generator=g).to(torch.bfloat16)
    wg = (torch.randn((F, Dm), generator=g) / Dm ** 0.5).to(torch.bfloat16)
    wu = (torch.randn((F, Dm), generator=g) / Dm ** 0.5).to(torch.bfloat16)
    wd = (torch.randn((Dm, F), generator=g) / F ** 0.5).to(torch.bfloat16)
    dy = (torch.randn((S, Dm), generator=g) / S).to(torch.bfloat16)
    x, wg, wu, wd, dy = (t.to(dev) for t in (x, wg, wu, wd, dy))

    def call():
        ws = torch.empty(up.upipe_mlp_workspace_bytes(S, Dm, F, tile, True), dtype=torch.uint8, device=dev)
        y = torch.full_like(x, float("nan"))
        up.upipe_mlp_tiled_fwd(x, wg, wu, wd, y, tile, ws)
        dx = torch.full((S, Dm), float("nan"), device=dev)
        dwg, dwu = (torch.full((F, Dm), float("nan"), device=dev) for _ in range(2))
        dwd = torch.full((Dm, F), float("nan"), device=dev)
        up.upipe_mlp_tiled_bwd(x, wg, wu, wd, dy, dx, dwg, dwu, dwd, tile, ws)
        torch.cuda.synchronize()
        return y, dx, dwg, dwu, dwd

    got = call()
    y, grads = swiglu_mlp(f64(x), f64(wg), f64(wu), f64(wd), f64(dy))
    assert_close("y", f64(got[0]), y, "bf16", per_item=True)
    for name, g_, r in zip(("dx", "dwg", "dwu", "dwd"), got[1:], grads):
        assert_close(name, f64(g_), r, "bf16", grad_scale=float(S), per_item=True,
                     elem_floor=1.0 if name == "dx" else "rms")
    for a, b in zip(got, call()):
        assert bit_equal(a, b), "repeated call differs"
