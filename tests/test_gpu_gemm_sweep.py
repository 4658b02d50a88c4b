"""A seeded random sweep of the bf16 MFMA GEMM (upipe_gemm_bf16) through the C
ABI against an fp64 product.

Each case draws M, N and K within the documented requirements (K a multiple
of 64, N a multiple of 8, M a multiple of 8 when A is M-contiguous), the
orientation of each operand, blocked layouts for the operands and for C
(block lengths that are powers of two from 8 to 128), C in bf16 or fp32, and
C += A B on fp32 C. About one case in five is large enough (at least one
256 x 256 tile per CU) to take the 8-wave kernel, the others the 128 x 128
kernel. The cases are fixed by one seed; each prints its shape first.
"""

import numpy as np
import pytest
import torch

import long_context_attention_upipe_amd as up
from gpu_util import f64

pytestmark = pytest.mark.gpu


def _draw_cases(n=30, seed=4242):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        a_k, b_k = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        big = rng.random() < 0.2
        if big:
            M, N, K = int(rng.integers(4096, 4400)), int(rng.integers(4096, 4400)), 64 * int(rng.integers(1, 5))
        else:
            M, N, K = int(rng.integers(1, 1500)), int(rng.integers(1, 1500)), 64 * int(rng.integers(1, 17))
        N = max(8, N // 8 * 8)
        if not a_k:
            M = max(8, M // 8 * 8)

        def blk_for(extent):
            if rng.random() >= 0.3:
                return None
            options = [b for b in (8, 16, 32, 64, 128) if extent % b == 0]
            return int(rng.choice(options)) if options else None

        a_blk = blk_for(K if a_k else M)
        b_blk = blk_for(K if b_k else N)
        c_blk = blk_for(N)
        c_fp32 = bool(rng.random() < 0.5)
        acc = c_fp32 and c_blk is None and rng.random() < 0.4
        cases.append((M, N, K, a_k, b_k, a_blk, b_blk, c_blk, c_fp32, acc, 9000 + i))
    return cases


CASES = _draw_cases()


def _id(c):
    M, N, K, a_k, b_k, a_blk, b_blk, c_blk, c_fp32, acc, _ = c
    blk = lambda b: f"/{b}" if b else ""  # noqa: E731
    return (f"{M}x{N}x{K}-a{'k' if a_k else 'm'}{blk(a_blk)}-b{'k' if b_k else 'n'}{blk(b_blk)}"
            f"-c{'f32' if c_fp32 else 'bf16'}{blk(c_blk)}{'-acc' if acc else ''}")


def _bf16(shape, seed, dev):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).to(dev)


def _operand(mat, kmajor, blk):
    """``mat`` [rows, K] stored as the layout says; returns (tensor, layout)."""
    R, K = mat.shape
    if kmajor:
        if blk is None:
            return mat.contiguous(), {"ld": K, "kmajor": 1}
        return mat.reshape(R, K // blk, blk).permute(1, 0, 2).contiguous(), \
            {"ld": blk, "kmajor": 1, "blk": blk, "blk_stride": R * blk}
    if blk is None:
        return mat.t().contiguous(), {"ld": R, "kmajor": 0}
    return mat.reshape(R // blk, blk, K).permute(0, 2, 1).contiguous(), \
        {"ld": blk, "kmajor": 0, "blk": blk, "blk_stride": K * blk}


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_gemm_matches_fp64(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    M, N, K, a_k, b_k, a_blk, b_blk, c_blk, c_fp32, acc, seed = case
    print(f"\n  gemm case {_id(case)}", flush=True)
    A, B = _bf16((M, K), seed, dev), _bf16((N, K), seed + 1, dev)
    ta, la = _operand(A, a_k, a_blk)
    tb, lb = _operand(B, b_k, b_blk)
    c_dtype = torch.float32 if c_fp32 else torch.bfloat16
    ref = f64(A) @ f64(B).T
    if c_blk is None:
        C = _bf16((M, N), seed + 2, dev).to(c_dtype) if acc else torch.full((M, N), float("nan"), dtype=c_dtype,
                                                                              device=dev)
        if acc:
            ref = ref + f64(C)
        up.upipe_gemm_bf16(ta, la, tb, lb, C, {"ld": N}, M, N, K, accumulate=acc)
        torch.cuda.synchronize()
        got = f64(C)
    else:
        C = torch.full((N // c_blk, M, c_blk), float("nan"), dtype=c_dtype, device=dev)
        up.upipe_gemm_bf16(ta, la, tb, lb, C, {"ld": c_blk, "blk": c_blk, "blk_stride": M * c_blk}, M, N, K)
        torch.cuda.synchronize()
        got = f64(C.permute(1, 0, 2).reshape(M, N))
    assert np.isfinite(got).all(), "an element of C was not written"
    rel = 1e-5 if c_fp32 else 5e-3
    err = np.abs(got - ref).max()
    print(f"    max |err| / max |ref| = {err / np.abs(ref).max():.2e}", flush=True)
    assert err <= rel * np.abs(ref).max()
