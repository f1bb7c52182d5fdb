"""GPU parity of the fused epilogue (dg_fp8_gemm_nt_epilogue; bjdmk.com.cn
DeepGEMM page s3.2: activation and residual fused into the GEMM's write-back;
pzsr.cn DeepGEMM page s2.3: SwiGLU).  Reference: the oracle's FP64 product of
the oracle's codes, then the oracle's FP64 epilogue; the GEMM tolerance
applies.  The shapes reach every store site: the 256 x 256 tile kernel, the
streaming small-M kernel, the LDS-ring small-M kernel without split-K and its
split-K reduction."""
import numpy as np
import pytest
import torch

import datagen
from gpu_util import assert_close, bf16_to_f64, dev, need_gpu, oracle_gemm_rows, tile_points

pytestmark = pytest.mark.gpu

ACTS = ["none", "relu", "silu", "gelu", "swiglu"]
# (M, N, K, workspace): tile kernel, streaming kernel, ring kernel, ring with split-K
SHAPES = [(300, 520, 640, False), (4, 1032, 1024, False), (40, 1032, 512, False),
          (12, 2056, 16384, True)]


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def operands(orc, M, N, K, seed):
    a = datagen.normal((M, K), 1.0, seed=seed, stream=0)
    b = datagen.normal((N, K), 0.05, seed=seed, stream=1)
    qa, sa = orc.quantize(a, 1)
    qb, sb = orc.quantize(b, 128)
    return qa, sa, qb, sb


def bf16_bits(x):
    """float array -> BF16 bits (round to nearest even), uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def run(dg, qa, sa, qb, sb, act, residual=None, in_place=False, ws=False):
    M, N = qa.shape[0], qb.shape[0]
    n_out = N // 2 if act == "swiglu" else N
    c = torch.full((M, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    res = None
    if residual is not None:
        res = torch.from_numpy(residual.view(np.int16)).cuda().view(torch.bfloat16)
        if in_place:
            c.copy_(res)
            res = c
    w = None
    if ws:
        nb = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, qa.shape[1])
        w = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
    dg.dg_fp8_gemm_nt_epilogue(c, dev(qa), dev(qb), dev(sa), dev(sb), 1, act=act, residual=res,
                               workspace=w)
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("M,N,K,ws", SHAPES)
@pytest.mark.parametrize("act", ACTS)
def test_epilogue_activations(dg, orc, M, N, K, ws, act):
    qa, sa, qb, sb = operands(orc, M, N, K, seed=M + N)
    ref = orc.epilogue(orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1), act)
    c = bf16_to_f64(run(dg, qa, sa, qb, sb, act, ws=ws))
    assert_close(c, ref, what="%s %dx%dx%d ws=%s" % (act, M, N, K, ws))


@pytest.mark.parametrize("M,N,K,ws", SHAPES)
@pytest.mark.parametrize("act", ["none", "silu", "swiglu"])
@pytest.mark.parametrize("in_place", [False, True])
def test_epilogue_residual(dg, orc, M, N, K, ws, act, in_place):
    qa, sa, qb, sb = operands(orc, M, N, K, seed=M * 3 + K)
    n_out = N // 2 if act == "swiglu" else N
    r = bf16_bits(datagen.normal((M, n_out), 0.5, seed=M, stream=7))
    ref = orc.epilogue(orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1), act, residual=r)
    c = bf16_to_f64(run(dg, qa, sa, qb, sb, act, residual=r, in_place=in_place, ws=ws))
    assert_close(c, ref, what="%s+res %dx%dx%d in_place=%s" % (act, M, N, K, in_place))


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_epilogue_tile_order_full_compare(dg, orc, act):
    """6 x 10 tiles of 256 x 256 (more than one 4-row band, every XCD's run
    of tiles, ragged edges) with the epilogue and a residual, in full."""
    M, N, K = 1300, 2312, 256
    qa, sa, qb, sb = operands(orc, M, N, K, seed=17)
    n_out = N // 2 if act == "swiglu" else N
    r = bf16_bits(datagen.normal((M, n_out), 0.5, seed=3, stream=7))
    ref = orc.epilogue(oracle_gemm_rows(orc, qa, sa, qb, sb, 1), act, residual=r)
    c = run(dg, qa, sa, qb, sb, act, residual=r)
    assert torch.isfinite(c).all()
    assert_close(bf16_to_f64(c), ref, what="%s+res tile order" % act)


@pytest.mark.parametrize("M,N,K,ws", SHAPES)
def test_epilogue_none_equals_plain_gemm(dg, orc, M, N, K, ws):
    qa, sa, qb, sb = operands(orc, M, N, K, seed=5)
    c1 = run(dg, qa, sa, qb, sb, "none", ws=ws)
    c2 = torch.empty_like(c1)
    w = None
    if ws:
        w = torch.zeros(max(dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K), 16), dtype=torch.uint8,
                        device="cuda")
    dg.dg_fp8_gemm_nt(c2, dev(qa), dev(qb), dev(sa), dev(sb), 1, workspace=w)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


def test_swiglu_full_size_sampled(dg, orc):
    """The MoE up-projection shape with gate and up interleaved (N = 2 x 11008),
    M = 2048 tokens, sampled against the oracle."""
    M, N, K = 2048, 22016, 4096
    qa, sa, qb, sb = operands(orc, M, N, K, seed=1)
    c = run(dg, qa, sa, qb, sb, "swiglu")
    assert torch.isfinite(c).all()                  # every element written (NaN prefill)
    g = np.random.default_rng(4)
    tm, tj = tile_points(M, N // 2, 256, 128, g)   # a 256 x 256 tile gives 128 outputs per row
    pm = np.concatenate([g.integers(0, M, 800), np.full(N // 2, M - 1), tm])
    pj = np.concatenate([g.integers(0, N // 2, 800), np.arange(N // 2), tj])
    assert pm.max() < M and pj.max() < N // 2
    gate = orc.gemm_nt_points(qa, sa, qb, sb, pm, 2 * pj, a_block_rows=1)
    up = orc.gemm_nt_points(qa, sa, qb, sb, pm, 2 * pj + 1, a_block_rows=1)
    ref = orc.epilogue(np.stack([gate, up], axis=1).reshape(1, -1), "swiglu")[0]
    got = c[torch.from_numpy(pm).cuda(), torch.from_numpy(pj).cuda()]
    rms = float(np.sqrt(np.mean(ref[:800] ** 2)))
    assert_close(got.float().cpu().numpy().astype(np.float64), ref, rms=rms, what="swiglu full")
