"""The bf16 MFMA GEMM and the chunked attention block (q, k, v projections
of each head chunk, attention, the chunk's share of the output projection;
forward and backward) through the C ABI, against the oracle."""

import math

import numpy as np
import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import OracleJobs, assert_close, bit_equal, f64, interleaved_parts
from long_context_attention_upipe_amd.workloads import make_block_inputs, sample_rows
from oracle.block import attention_block_backward, attention_block_forward, attention_block_rows

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _bf16(shape, seed, dev, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).to(dev)


def _as_operand(mat, kmajor, blk=None):
    """Store the logical operand ``mat`` [rows, K] (rows = M or N) in the
    layout the GEMM is told about; returns (tensor, layout)."""
    R, K = mat.shape
    if kmajor:
        if blk is None:
            return mat.contiguous(), {"ld": K, "kmajor": 1}
        t = mat.reshape(R, K // blk, blk).permute(1, 0, 2).contiguous()  # [K/blk][R][blk]
        return t, {"ld": blk, "kmajor": 1, "blk": blk, "blk_stride": R * blk}
    if blk is None:
        return mat.t().contiguous(), {"ld": R, "kmajor": 0}
    t = mat.reshape(R // blk, blk, K).permute(0, 2, 1).contiguous()  # [R/blk][K][blk]
    return t, {"ld": blk, "kmajor": 0, "blk": blk, "blk_stride": K * blk}


@pytest.mark.parametrize("a_kmajor,b_kmajor", [(1, 1), (1, 0), (0, 1), (0, 0)])
@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16])
def test_gemm_every_layout(a_kmajor, b_kmajor, c_dtype):
    """C = A B^T-stored for every pair of operand layouts; ragged M and N
    (not multiples of the 128 x 128 tile), K over several 64-deep steps."""
    dev = _dev()
    M, N, K = 264, 200, 192
    A, B = _bf16((M, K), 1, dev), _bf16((N, K), 2, dev)
    ta, la = _as_operand(A, a_kmajor)
    tb, lb = _as_operand(B, b_kmajor)
    C = torch.full((M, N), float("nan"), dtype=c_dtype, device=dev)
    up.upipe_gemm_bf16(ta, la, tb, lb, C, {"ld": N}, M, N, K)
    torch.cuda.synchronize()
    ref = f64(A) @ f64(B).T
    rel = 1e-5 if c_dtype == torch.float32 else 5e-3
    assert_close("C", f64(C), ref, "bf16" if c_dtype == torch.bfloat16 else "fp32", rel_only=True)
    assert np.abs(f64(C) - ref).max() <= rel * np.abs(ref).max()


def test_gemm_blocked_operands_and_output_and_accumulate():
    """Blocked layouts (a head-major [heads][S][d] buffer read as one
    [S][heads*d] matrix, and written the same way), then C += A B on fp32 C;
    M ragged and not a multiple of 8 (a k-major A allows it)."""
    dev = _dev()
    M, N, K = 1001, 256, 256
    A, B = _bf16((M, K), 3, dev), _bf16((N, K), 4, dev, 0.1)
    ta, la = _as_operand(A, 1, blk=64)
    tb, lb = _as_operand(B, 0, blk=128)
    C = torch.empty((N // 128, M, 128), dtype=torch.bfloat16, device=dev)  # [N/128][M][128]
    up.upipe_gemm_bf16(ta, la, tb, lb, C, {"ld": 128, "blk": 128, "blk_stride": M * 128}, M, N, K)
    ref = f64(A) @ f64(B).T
    got = f64(C.permute(1, 0, 2).reshape(M, N))
    assert np.abs(got - ref).max() <= 5e-3 * np.abs(ref).max()
    C0 = _bf16((M, N), 5, dev).float()
    C1 = C0.clone()
    up.upipe_gemm_bf16(ta, la, tb, lb, C1, {"ld": N}, M, N, K, accumulate=True)
    torch.cuda.synchronize()
    ref1 = f64(C0) + ref
    assert np.abs(f64(C1) - ref1).max() <= 1e-5 * np.abs(ref1).max()


@pytest.mark.parametrize("a_kmajor,b_kmajor", [(1, 1), (1, 0), (0, 1), (0, 0)])
@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16])
def test_gemm_256_tiles_every_layout_and_same_sums_as_128_tiles(a_kmajor, b_kmajor, c_dtype):
    """Problems with at least one 256 x 256 tile per CU take the 8-wave
    kernel: every layout pair, ragged M and N, K over several steps, against
    fp64; and, since both kernels add each C entry over K in the same order,
    the first 256 rows equal (bit for bit) a 256-row product, which takes the
    128 x 128 kernel."""
    dev = _dev()
    M, N, K = 4104, 4000, 320  # 17 x 16 tiles of 256
    print(f"\n  gemm {M}x{N}x{K} a_kmajor={a_kmajor} b_kmajor={b_kmajor} {c_dtype}", flush=True)
    A, B = _bf16((M, K), 11, dev), _bf16((N, K), 12, dev)
    ta, la = _as_operand(A, a_kmajor)
    tb, lb = _as_operand(B, b_kmajor)
    C = torch.full((M, N), float("nan"), dtype=c_dtype, device=dev)
    up.upipe_gemm_bf16(ta, la, tb, lb, C, {"ld": N}, M, N, K)
    A_top = A[:256]
    ta2, la2 = _as_operand(A_top, a_kmajor)
    C2 = torch.full((256, N), float("nan"), dtype=c_dtype, device=dev)
    up.upipe_gemm_bf16(ta2, la2, tb, lb, C2, {"ld": N}, 256, N, K)
    torch.cuda.synchronize()
    ref = f64(A) @ f64(B).T
    rel = 1e-5 if c_dtype == torch.float32 else 5e-3
    got = f64(C)
    assert np.isfinite(got).all()
    assert np.abs(got - ref).max() <= rel * np.abs(ref).max()
    assert bit_equal(C[:256], C2), "256 x 256 and 128 x 128 tiles sum differently"


def test_gemm_256_tiles_blocked_operands_and_output_and_accumulate():
    """The 8-wave kernel with blocked layouts (k-major A in 64-element blocks,
    mn-major B in 128-element blocks, C written in 128-column blocks), M not a
    multiple of 8, then C += A B on fp32 C."""
    dev = _dev()
    M, N, K = 4353, 3840, 256  # 18 x 15 tiles of 256
    A, B = _bf16((M, K), 13, dev), _bf16((N, K), 14, dev, 0.1)
    ta, la = _as_operand(A, 1, blk=64)
    tb, lb = _as_operand(B, 0, blk=128)
    C = torch.empty((N // 128, M, 128), dtype=torch.bfloat16, device=dev)
    up.upipe_gemm_bf16(ta, la, tb, lb, C, {"ld": 128, "blk": 128, "blk_stride": M * 128}, M, N, K)
    ref = f64(A) @ f64(B).T
    got = f64(C.permute(1, 0, 2).reshape(M, N))
    assert np.abs(got - ref).max() <= 5e-3 * np.abs(ref).max()
    C0 = _bf16((M, N), 15, dev).float()
    C1 = C0.clone()
    up.upipe_gemm_bf16(ta, la, tb, lb, C1, {"ld": N}, M, N, K, accumulate=True)
    torch.cuda.synchronize()
    ref1 = f64(C0) + ref
    assert np.abs(f64(C1) - ref1).max() <= 1e-5 * np.abs(ref1).max()


def test_gemm_rejects_bad_layouts():
    dev = _dev()
    A, B = _bf16((64, 100), 6, dev), _bf16((64, 100), 7, dev)
    C = torch.empty((64, 64), device=dev)
    with pytest.raises(up.UpipeError, match="multiple of 64"):
        up.upipe_gemm_bf16(A, {"ld": 100, "kmajor": 1}, B, {"ld": 100, "kmajor": 1}, C, {"ld": 64}, 64, 64, 100)
    A = _bf16((64, 128), 8, dev)
    with pytest.raises(up.UpipeError, match="beyond the tensor"):
        up.upipe_gemm_bf16(A, {"ld": 128, "kmajor": 1}, A, {"ld": 128, "kmajor": 1}, C, {"ld": 64}, 64, 65 + 7,
                           128)


def _block_run(x, wq, wk, wv, wo, Hq, Hkv, hc, causal=True, keep_out=True):
    S, Dm = x.shape
    d = wq.shape[0] // Hq
    ws = torch.empty(up.upipe_attn_block_fwd_workspace_bytes(S, Dm, Hq, Hkv, d, hc), dtype=torch.uint8,
                     device=x.device)
    y = torch.empty((S, Dm), dtype=torch.float32, device=x.device)
    out = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=x.device) if keep_out else None
    lse = torch.empty((Hq, S), dtype=torch.float32, device=x.device)
    up.upipe_attn_block_fwd(x, wq, wk, wv, wo, y, out, lse, Hq, Hkv, hc, causal, ws)
    torch.cuda.synchronize()
    return y, out, lse


@pytest.mark.parametrize("S,Dm,Hq,Hkv,d,hcs,causal", [
    (1, 64, 2, 1, 64, (1, 2), True),
    (300, 512, 4, 1, 128, (1, 2, 4), True),
    (1000, 192, 8, 2, 64, (1, 2, 4, 8), True),
    (517, 256, 4, 2, 128, (1, 4), False),
])
def test_block_forward_full(S, Dm, Hq, Hkv, d, hcs, causal):
    dev = _dev()
    print(f"\n  block S={S} Dm={Dm} Hq={Hq} Hkv={Hkv} d={d} causal={causal} head_chunks={hcs}", flush=True)
    x, wq, wk, wv, wo = make_block_inputs(S, Dm, Hq, Hkv, d, seed=40 + S, device=dev)
    y_ref, o_ref, l_ref = attention_block_forward(*(f64(t) for t in (x, wq, wk, wv, wo)), Hq, Hkv, causal=causal)
    first = None
    for hc in hcs:
        print(f"   head_chunk={hc}", flush=True)
        r = _block_run(x, wq, wk, wv, wo, Hq, Hkv, hc, causal)
        assert_close("y", f64(r[0]), y_ref, "bf16", per_item=True)
        assert_close("out", f64(r[1]), o_ref, "bf16", per_item=True)
        assert_close("lse", f64(r[2]), l_ref, "bf16")
        if first is None:
            first = r
        else:
            for name, a, b in zip(("y", "out", "lse"), r, first):
                assert bit_equal(a, b), f"{name} differs between head_chunk {hcs[0]} and {hc}"


@pytest.mark.slow
def test_block_forward_128k_sampled_rows():
    """131,072 tokens, the 8B share's heads (Hq = 4, Hkv = 1, d = 128) with
    Dm = 512: y, out and lse at 1024 sampled rows (the oracle's k and v over
    the whole sequence, q and attention at the rows), head_chunk 1, 2, 4
    bit-identical; y is also written without out (out = NULL) and agrees."""
    dev = _dev()
    S, Dm, Hq, Hkv, d = 131072, 512, 4, 1, 128
    x, wq, wk, wv, wo = make_block_inputs(S, Dm, Hq, Hkv, d, seed=9000, device=dev)
    rows = sample_rows(S, 1024, seed=9007)
    xs, wqs, wks, wvs, wos = (f64(t) for t in (x, wq, wk, wv, wo))
    with OracleJobs() as jobs:
        parts = interleaved_parts(len(rows), 32)
        job = jobs.map(lambda p: attention_block_rows(xs, wqs, wks, wvs, wos, Hq, Hkv, rows[p]), parts, "block rows")
        first = None
        for hc in (1, 2, 4):
            print(f"   head_chunk={hc}", flush=True)
            r = _block_run(x, wq, wk, wv, wo, Hq, Hkv, hc)
            if first is None:
                first = r
            else:
                for name, a, b in zip(("y", "out", "lse"), r, first):
                    assert bit_equal(a, b), f"{name} differs between head_chunk 1 and {hc}"
                del r
        y2 = _block_run(x, wq, wk, wv, wo, Hq, Hkv, 2, keep_out=False)[0]
        assert bit_equal(y2, first[0]), "y differs when out is not kept"
        y_ref, o_ref, l_ref = np.empty((len(rows), Dm)), np.empty((len(rows), Hq, d)), np.empty((Hq, len(rows)))
        for p, (yy, oo, ll) in zip(parts, jobs.gather(job)):
            y_ref[p], o_ref[p], l_ref[:, p] = yy, oo, ll
    rows_t = torch.from_numpy(rows).to(dev)
    assert_close("y", f64(first[0][rows_t]), y_ref, "bf16", per_item=True)
    assert_close("out", f64(first[1][rows_t]), o_ref, "bf16", per_item=True)
    assert_close("lse", f64(first[2][:, rows_t]), l_ref, "bf16")
    # the block's peak device memory without out: pool (grows with head_chunk) + x, weights, y, lse
    pools = [up.upipe_attn_block_fwd_workspace_bytes(S, Dm, Hq, Hkv, d, hc) for hc in (1, 2, 4)]
    assert pools[0] < pools[1] < pools[2]
    print(f"   pools (GiB) at head_chunk 1/2/4: {[round(p / 2 ** 30, 3) for p in pools]}", flush=True)
    assert math.isfinite(float(first[0].abs().max()))


GRADS = ("dx", "dwq", "dwk", "dwv", "dwo")


def _block_bwd_run(x, wq, wk, wv, wo, dy, Hq, Hkv, hc, causal=True, out=None, lse=None):
    S, Dm = x.shape
    d = wq.shape[0] // Hq
    ws = torch.empty(up.upipe_attn_block_bwd_workspace_bytes(S, Dm, Hq, Hkv, d, hc, out is None),
                     dtype=torch.uint8, device=x.device)
    # NaN-filled outputs: an element the library does not write fails the check
    res = [torch.full(t.shape, float("nan"), dtype=torch.float32, device=x.device) for t in (x, wq, wk, wv, wo)]
    up.upipe_attn_block_bwd(x, wq, wk, wv, wo, dy, out, lse, *res, Hq, Hkv, hc, causal, ws)
    torch.cuda.synchronize()
    return res


def _check_grads(got, refs):
    """Element bounds: dx per token row (an early key's dk and dv sum over
    every later row, so its token's dx row is far larger than the typical
    one and carries proportionally larger bf16 rounding), the weight
    gradients (sums over all tokens) against the tensor's RMS."""
    for name, g, ref in zip(GRADS, got, refs):
        assert_close(name, f64(g), ref, "bf16", per_item=True, elem_floor="row" if name == "dx" else "rms")


@pytest.mark.parametrize("S,Dm,Hq,Hkv,d,hcs,causal", [
    (1, 64, 2, 1, 64, (1, 2), True),
    (300, 512, 4, 1, 128, (1, 2, 4), True),
    (1000, 192, 8, 2, 64, (1, 2, 4, 8), True),
    (517, 256, 4, 2, 128, (1, 4), False),
    (8192, 256, 4, 1, 128, (1, 4), True),
    # 20,000 tokens: the weight gradients' token contraction runs split in two
    # ranges (added in order by a second kernel), then the 32-token tail
    (20000, 128, 2, 1, 64, (1, 2), True),
])
def test_block_backward_full(S, Dm, Hq, Hkv, d, hcs, causal):
    """dx and the four weight gradients against the oracle at every element,
    with o recomputed (out = None) at each head_chunk (bit-identical across
    them) and with the forward's out and lse handed over; the token
    contraction's ragged last step (S not a multiple of 64) included."""
    dev = _dev()
    print(f"\n  block backward S={S} Dm={Dm} Hq={Hq} Hkv={Hkv} d={d} causal={causal} head_chunks={hcs}", flush=True)
    x, wq, wk, wv, wo = make_block_inputs(S, Dm, Hq, Hkv, d, seed=60 + S, device=dev)
    dy = _bf16((S, Dm), 61 + S, dev)
    refs = attention_block_backward(*(f64(t) for t in (x, wq, wk, wv, wo, dy)), Hq, Hkv, causal=causal)
    first = None
    for hc in hcs:
        print(f"   head_chunk={hc} (o recomputed)", flush=True)
        r = _block_bwd_run(x, wq, wk, wv, wo, dy, Hq, Hkv, hc, causal)
        _check_grads(r, refs)
        if first is None:
            first = r
        else:
            for name, a, b in zip(GRADS, r, first):
                assert bit_equal(a, b), f"{name} differs between head_chunk {hcs[0]} and {hc}"
    print(f"   head_chunk={hcs[-1]} (out and lse from the forward)", flush=True)
    _, out, lse = _block_run(x, wq, wk, wv, wo, Hq, Hkv, hcs[-1], causal)
    r = _block_bwd_run(x, wq, wk, wv, wo, dy, Hq, Hkv, hcs[-1], causal, out=out, lse=lse)
    _check_grads(r, refs)
    # dWo = dy^T o reads the same o bits either way
    assert bit_equal(r[4], first[4]), "dwo differs between recomputed and handed-over o"
