"""The sequence-tiled SwiGLU MLP through the C ABI, against the oracle: y,
dx and the weight gradients, ragged last tiles, and results that do not
depend on the tile size (y, dx bit for bit; the weight gradients up to their
summation order)."""

import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import assert_close, bit_equal, f64
from oracle.mlp import swiglu_mlp

pytestmark = pytest.mark.gpu


def _inputs(S, Dm, F, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((S, Dm), generator=g).to(torch.bfloat16)
    wg = (torch.randn((F, Dm), generator=g) / Dm ** 0.5).to(torch.bfloat16)
    wu = (torch.randn((F, Dm), generator=g) / Dm ** 0.5).to(torch.bfloat16)
    wd = (torch.randn((Dm, F), generator=g) / F ** 0.5).to(torch.bfloat16)
    dy = (torch.randn((S, Dm), generator=g) / S).to(torch.bfloat16)  # a loss averaged over S tokens
    return [t.to(dev) for t in (x, wg, wu, wd, dy)]


def _run(x, wg, wu, wd, dy, tile):
    S, Dm = x.shape
    F = wg.shape[0]
    ws = torch.empty(up.upipe_mlp_workspace_bytes(S, Dm, F, tile, True), dtype=torch.uint8, device=x.device)
    y = torch.full_like(x, float("nan"))
    up.upipe_mlp_tiled_fwd(x, wg, wu, wd, y, tile, ws)
    dx = torch.full((S, Dm), float("nan"), device=x.device)
    dwg, dwu = (torch.full((F, Dm), float("nan"), device=x.device) for _ in range(2))
    dwd = torch.full((Dm, F), float("nan"), device=x.device)
    up.upipe_mlp_tiled_bwd(x, wg, wu, wd, dy, dx, dwg, dwu, dwd, tile, ws)
    torch.cuda.synchronize()
    return y, dx, dwg, dwu, dwd


@pytest.mark.parametrize("S,Dm,F,tile", [
    (1, 64, 64, 64),
    (300, 128, 192, 128),     # ragged last tile (44 tokens)
    (1000, 256, 512, 256),
    (4096, 512, 1408, 1024),
])
def test_tiled_mlp_matches_oracle(S, Dm, F, tile):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    print(f"\n  S={S} Dm={Dm} F={F} tile={tile}", flush=True)
    x, wg, wu, wd, dy = _inputs(S, Dm, F, 300 + S, dev)
    got = _run(x, wg, wu, wd, dy, tile)
    y, grads = swiglu_mlp(f64(x), f64(wg), f64(wu), f64(wd), f64(dy))
    assert_close("y", f64(got[0]), y, "bf16", per_item=True)
    for name, g_, r in zip(("dx", "dwg", "dwu", "dwd"), got[1:], grads):
        # gradients at unit upstream scale (dy was drawn as N(0,1)/S); the
        # weight gradients sum over every token: element floor = their RMS
        assert_close(name, f64(g_), r, "bf16", grad_scale=float(S), per_item=True,
                     elem_floor=1.0 if name == "dx" else "rms")


def test_tiled_mlp_tile_size_changes_only_weight_gradient_order():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    x, wg, wu, wd, dy = _inputs(2000, 256, 512, 7, dev)
    a = _run(x, wg, wu, wd, dy, 256)
    b = _run(x, wg, wu, wd, dy, 1024)
    assert bit_equal(a[0], b[0]) and bit_equal(a[1], b[1])
    for p, q in zip(a[2:], b[2:]):
        assert float((p - q).abs().max()) <= 1e-5 * float(p.abs().max())
    c = _run(x, wg, wu, wd, dy, 256)
    for p, q in zip(a, c):
        assert bit_equal(p, q), "repeated call differs"
