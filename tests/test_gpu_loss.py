"""The sequence-tiled cross-entropy through the C ABI, against the oracle:
loss per token, dh and dW, ragged last tiles, ignored labels, forward-only
calls, and results that do not depend on the tile size beyond dW's
summation order."""

import numpy as np
import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import assert_close, bit_equal, f64
from oracle.loss import cross_entropy

pytestmark = pytest.mark.gpu


def _inputs(S, Dm, V, seed, dev, ignore_every=0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    h = torch.randn((S, Dm), generator=g).to(torch.bfloat16)
    w = (torch.randn((V, Dm), generator=g) / Dm ** 0.5 * 2).to(torch.bfloat16)
    labels = torch.randint(0, V, (S,), generator=g, dtype=torch.int32)
    if ignore_every:
        labels[::ignore_every] = -100
    return h.to(dev), w.to(dev), labels.to(dev)


def _run(h, w, labels, tile, scale, grad=True):
    S, Dm = h.shape
    V = w.shape[0]
    ws = torch.empty(up.upipe_ce_loss_workspace_bytes(S, Dm, V, tile, grad), dtype=torch.uint8, device=h.device)
    loss = torch.full((S,), float("nan"), device=h.device)
    dh = torch.full_like(h, float("nan")) if grad else None
    dw = torch.full((V, Dm), float("nan"), device=h.device) if grad else None
    up.upipe_ce_loss_tiled(h, w, labels, loss, dh, dw, tile, scale, ws)
    torch.cuda.synchronize()
    return loss, dh, dw


@pytest.mark.parametrize("S,Dm,V,tile,ignore_every", [
    (1, 64, 8, 64, 0),
    (300, 128, 1000, 128, 7),      # ragged last tile (44 tokens), V not a multiple of 64
    (1000, 256, 5000, 256, 0),
    (4096, 512, 32000, 1024, 13),
])
def test_tiled_cross_entropy_matches_oracle(S, Dm, V, tile, ignore_every):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    print(f"\n  S={S} Dm={Dm} V={V} tile={tile}", flush=True)
    h, w, labels = _inputs(S, Dm, V, 100 + S, dev, ignore_every)
    n = int((labels >= 0).sum().item())
    scale = 1.0 / max(1, n)
    loss, dh, dw = _run(h, w, labels, tile, scale)
    rl, rdh, rdw = cross_entropy(f64(h), f64(w), labels.cpu().numpy(), scale=scale)
    assert_close("loss", f64(loss), rl, "bf16", per_item=False)
    # gradients at unit upstream scale (x N), as for attention's dO
    assert_close("dh", f64(dh), rdh, "bf16", grad_scale=float(n), per_item=True)
    assert_close("dw", f64(dw), rdw, "bf16", grad_scale=float(n), per_item=True, elem_floor="row")
    lf, _, _ = _run(h, w, labels, tile, scale, grad=False)
    assert bit_equal(lf, loss), "forward-only loss differs from the loss with gradients"
    if ignore_every:
        assert float(loss[labels < 0].abs().max()) == 0.0
        assert float(dh[labels < 0].float().abs().max()) == 0.0


def test_tiled_cross_entropy_tile_size_changes_only_dw_order():
    """loss and dh are per token: bit-identical for any tile size; dW sums
    over tiles, so it agrees to rounding."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    h, w, labels = _inputs(2000, 256, 4096, 7, dev)
    a = _run(h, w, labels, 256, 1e-3)
    b = _run(h, w, labels, 1024, 1e-3)
    assert bit_equal(a[0], b[0]) and bit_equal(a[1], b[1])
    assert float((a[2] - b[2]).abs().max()) <= 1e-5 * float(a[2].abs().max())
    c = _run(h, w, labels, 256, 1e-3)
    for x, y in zip(a, c):
        assert bit_equal(x, y), "repeated call differs"


def test_label_out_of_range_poisons_its_row_and_nothing_else():
    """A label >= V names no logit. The kernel reads nothing for it: that
    token's loss is NaN, and so are its dh row and (as dW sums over every
    token) all of dW. Every other token's loss and dh row are bit-identical
    to a call with that token's label ignored."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    S, Dm, V, tile = 300, 128, 1000, 128
    h, w, labels = _inputs(S, Dm, V, 11, dev)
    bad, ignored = labels.clone(), labels.clone()
    for r in (0, 130, 299):  # first row, a row of the second tile, the last row of the ragged tile
        bad[r] = V + 3 * r
        ignored[r] = -100
    print(f"\n  S={S} V={V}: labels out of range at rows 0, 130, 299", flush=True)
    loss_b, dh_b, dw_b = _run(h, w, bad, tile, 1e-2)
    loss_i, dh_i, _ = _run(h, w, ignored, tile, 1e-2)
    rows = torch.tensor([0, 130, 299], device=dev)
    keep = torch.ones(S, dtype=torch.bool, device=dev)
    keep[rows] = False
    assert bool(torch.isnan(loss_b[rows]).all()) and bool(torch.isnan(dh_b[rows].float()).all())
    assert bool(torch.isnan(dw_b).all())
    assert bit_equal(loss_b[keep], loss_i[keep]) and bit_equal(dh_b[keep], dh_i[keep])
