"""GPU parity of the fused epilogue on the grouped GEMMs (bjdmk.com.cn
DeepGEMM page s3.2: activation and residual fused into the write-back;
pzsr.cn DeepGEMM page s2.3: SwiGLU inside the MoE kernel).  Reference: the
oracle's grouped FP64 product, then the oracle's FP64 epilogue, on real /
valid rows; the GEMM tolerance applies.  Contiguous layout: padding rows
(and whole padding blocks) must be exact zeros, also with SwiGLU's half-width
output.  Masked layout: rows past the counts keep their sentinel bits."""
import numpy as np
import pytest
import torch

import datagen
from gpu_util import assert_close, bf16_to_f64, dev, need_gpu, tile_points

pytestmark = pytest.mark.gpu

ACTS = ["relu", "silu", "gelu", "swiglu"]
SENTINEL = 0x4B1D


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def contig_operands(orc, tokens, G, N, K, seed):
    r = datagen.moe_routing(tokens, G, 2, align=128, seed=seed)
    mi = r["m_indices"]
    # one whole 128-row block of padding at the end
    mi = np.concatenate([mi, np.full(128, -1, np.int32)])
    row_token = np.concatenate([r["row_token"], np.full(128, -1, np.int64)])
    a = datagen.gather_rows(datagen.normal((tokens, K), 1.0, seed=seed, stream=1), row_token)
    qa, sa = orc.quantize(a, 1)
    w = datagen.normal((G * N, K), 0.05, seed=seed, stream=2)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, N // 128), np.float32)
    for e in range(G):
        qb[e], sb[e] = orc.quantize(w[e * N:(e + 1) * N], 128)
    return qa, sa, qb, sb, mi


@pytest.mark.parametrize("residual", ["none", "separate", "in_place"])
@pytest.mark.parametrize("act", ACTS)
def test_grouped_contig_epilogue(dg, orc, act, residual):
    tokens, G, N, K = 200, 4, 512, 384
    qa, sa, qb, sb, mi = contig_operands(orc, tokens, G, N, K, seed=21)
    M = qa.shape[0]
    n_out = N // 2 if act == "swiglu" else N
    res_bits = None
    c = torch.full((M, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    res = None
    if residual != "none":
        res_bits = bf16_bits(datagen.normal((M, n_out), 0.5, seed=22, stream=0))
        res = torch.from_numpy(res_bits.view(np.int16)).cuda().view(torch.bfloat16)
        if residual == "in_place":
            c.copy_(res)
            res = c
    dg.dg_fp8_grouped_gemm_contig(c, dev(qa), dev(qb), dev(sa), dev(sb), 1, dev(mi), act=act,
                                  residual=res)
    torch.cuda.synchronize()
    got = bf16_to_f64(c)
    real = mi >= 0
    assert np.all(got[~real] == 0.0), "padding rows must be zeros"
    acc = orc.grouped_gemm_contig(qa, sa, qb, sb, mi, a_block_rows=1)
    ref = orc.epilogue(acc[real], act, None if res_bits is None else res_bits[real])
    assert_close(got[real], ref, what="grouped epilogue %s/%s" % (act, residual))


def test_grouped_contig_no_epilogue_is_the_plain_call(dg, orc):
    qa, sa, qb, sb, mi = contig_operands(orc, 200, 4, 512, 384, seed=23)
    M, N = qa.shape[0], qb.shape[1]
    c1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    A, B, SA, SB, MI = dev(qa), dev(qb), dev(sa), dev(sb), dev(mi)
    dg.lib.dg_fp8_grouped_gemm_contig_epilogue(c1.data_ptr(), A.data_ptr(), B.data_ptr(),
                                               SA.data_ptr(), SB.data_ptr(), 1, MI.data_ptr(),
                                               4, M, N, qa.shape[1], 0, None, None)
    dg.dg_fp8_grouped_gemm_contig(c2, A, B, SA, SB, 1, MI)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_grouped_swiglu_moe_shape_sampled(dg, orc):
    """8 experts, 1024 tokens top-2, gate/up interleaved 2 x 2048 rows per
    expert, K 4096: SwiGLU fused, 3000 sampled outputs."""
    G, tokens, N, K = 8, 1024, 4096, 4096
    r = datagen.moe_routing(tokens, G, 2, align=128, seed=0)
    mi = r["m_indices"]
    a = datagen.gather_rows(datagen.normal((tokens, K), 1.0, seed=0, stream=1), r["row_token"])
    qa, sa = orc.quantize(a, 1)
    w = datagen.normal((G * N, K), 0.02, seed=0, stream=2)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, N // 128), np.float32)
    for e in range(G):
        qb[e], sb[e] = orc.quantize(w[e * N:(e + 1) * N], 128)
    M = qa.shape[0]
    c = torch.full((M, N // 2), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_grouped_gemm_contig(c, dev(qa), dev(qb), dev(sa), dev(sb), 1, dev(mi), act="swiglu")
    torch.cuda.synchronize()
    got = bf16_to_f64(c)
    assert np.all(np.isfinite(got))                 # every element written (NaN prefill)
    assert np.all(got[mi < 0] == 0.0)
    rng = np.random.default_rng(5)
    tm, tj = tile_points(M, N // 2, 128, 128, rng, rows=np.nonzero(mi >= 0)[0])
    pm = np.concatenate([rng.choice(np.nonzero(mi >= 0)[0], 3000), tm])
    pj = np.concatenate([rng.integers(0, N // 2, 3000), tj])
    acc = np.empty((pm.size, 2))
    for e in range(G):
        sel = mi[pm] == e
        for h in range(2):   # gate (column 2j) and up (2j + 1)
            acc[sel, h] = orc.gemm_nt_points(qa, sa, qb[e], sb[e], pm[sel], 2 * pj[sel] + h,
                                             a_block_rows=1)
    ref = orc.epilogue(acc, "swiglu")[:, 0]
    assert_close(got[pm, pj], ref, what="grouped SwiGLU MoE")


def masked_operands(orc, G, max_m, N, K, seed):
    qa = np.empty((G, max_m, K), np.uint8)
    sa = np.empty((G, K // 128, max_m), np.float32)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, -(-N // 128)), np.float32)
    for g in range(G):
        qa[g], sa[g] = orc.quantize(datagen.normal((max_m, K), 1.0, seed=seed, stream=2 * g), 1)
        qb[g], sb[g] = orc.quantize(datagen.normal((N, K), 0.05, seed=seed, stream=2 * g + 1), 128)
    return qa, sa, qb, sb


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("act,residual", [("swiglu", True), ("gelu", False), ("relu", True),
                                          ("silu", False)])
def test_masked_epilogue(dg, orc, act, residual, ws):
    G, max_m, N, K = 6, 24, 1024, 4096
    mm = np.array([24, 0, 7, 13, 1, 24], np.int32)
    qa, sa, qb, sb = masked_operands(orc, G, max_m, N, K, seed=31)
    n_out = N // 2 if act == "swiglu" else N
    c = torch.full((G, max_m, n_out), SENTINEL, dtype=torch.int16, device="cuda")
    res_bits, res = None, None
    if residual:
        res_bits = bf16_bits(datagen.normal((G, max_m, n_out), 0.5, seed=32, stream=0))
        res = torch.from_numpy(res_bits.view(np.int16)).cuda()
    w = None
    if ws:
        nb = dg.dg_fp8_grouped_gemm_masked_workspace_bytes(G, max_m, N, K)
        assert nb > 0
        w = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    dg.dg_fp8_grouped_gemm_masked(c, dev(qa), dev(qb), dev(sa), dev(sb), 1, dev(mm), workspace=w,
                                  act=act, residual=res)
    torch.cuda.synchronize()
    bits = c.cpu().numpy().view(np.uint16)
    got = bf16_to_f64(c)
    acc = orc.grouped_gemm_masked(qa, sa, qb, sb, mm, a_block_rows=1)
    for g in range(G):
        assert np.all(bits[g, mm[g]:] == SENTINEL), "rows past the count were written"
        if mm[g] == 0:
            continue
        ref = orc.epilogue(acc[g, :mm[g]], act, None if res_bits is None else res_bits[g, :mm[g]])
        assert_close(got[g, :mm[g]], ref, what="masked epilogue %s g%d" % (act, g))
