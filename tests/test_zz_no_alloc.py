"""dg_fp8_gemm_nt_noalloc: the GEMM entry point that allocates nothing (its
split-K scratch is the library's static per-GPU array).  Called through the
C ABI, its output must equal dg_fp8_gemm_nt's with a caller workspace bit for
bit (same plan, same summation order) and meet the GEMM tolerance against
the oracle, on consecutive calls whose second input is smaller than the
first (the array keeps the previous call's contents)."""
import numpy as np
import pytest
import torch

import datagen
from gpu_util import assert_close, bf16_to_f64, dev, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def operands(orc, M, N, K, seed):
    qa, sa = orc.quantize(datagen.normal((M, K), 1.0, seed=seed, stream=0), 1)
    qb, sb = orc.quantize(datagen.normal((N, K), 0.02, seed=seed, stream=1), 128)
    return qa, sa, qb, sb


def with_workspace(dg, ops, M, N, K):
    a, sa, b, sb = ops
    nb = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    ws = dg.alloc_workspace(nb) if nb else None
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm_nt(c, a, b, sa, sb, 1, workspace=ws)
    torch.cuda.synchronize()
    return c


def test_noalloc_matches_the_workspace_call_on_consecutive_calls(dg, orc):
    # split-K plans (LDS-ring kernel): 64 x 7168 x 2048 (2 splits), then a
    # smaller 33 x 2048 x 1024 (2 splits, fewer tiles); then one that splits
    # more (16 x 4096 x 8192) and a plan with no scratch at all (256 rows)
    shapes = [(64, 7168, 2048), (33, 2048, 1024), (12, 7168, 16384), (256, 512, 384)]
    for i, (M, N, K) in enumerate(shapes):
        qa, sa, qb, sb = operands(orc, M, N, K, seed=40 + i)
        ops = (dev(qa), dev(sa), dev(qb), dev(sb))
        if i < 3:
            assert dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K) > dg.WORKSPACE_COUNTER_BYTES
        assert dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K) <= dg.NOALLOC_SCRATCH_BYTES
        want = with_workspace(dg, ops, M, N, K)
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        a, sa_d, b, sb_d = ops
        dg.dg_fp8_gemm_nt_noalloc(c, a, b, sa_d, sb_d, 1)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), want.view(torch.int16)), (M, N, K)
        ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1)
        assert_close(bf16_to_f64(c), ref, what="noalloc %dx%dx%d" % (M, N, K))


def test_noalloc_repeated_calls_stay_identical(dg, orc):
    """The counters the previous call left in the array are cleared, and a
    call on a side stream of the current device works too."""
    M, N, K = 16, 7168, 8192                        # 8 splits on the LDS-ring kernel
    assert dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K) > dg.WORKSPACE_COUNTER_BYTES
    qa, sa, qb, sb = operands(orc, M, N, K, seed=50)
    a, sa_d, b, sb_d = dev(qa), dev(sa), dev(qb), dev(sb)
    want = with_workspace(dg, (a, sa_d, b, sb_d), M, N, K)
    side = torch.cuda.Stream()
    for rep in range(3):
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        if rep == 2:
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                dg.dg_fp8_gemm_nt_noalloc(c, a, b, sa_d, sb_d, 1)
        else:
            dg.dg_fp8_gemm_nt_noalloc(c, a, b, sa_d, sb_d, 1)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), want.view(torch.int16)), rep
