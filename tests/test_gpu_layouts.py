"""GPU parity of the training layouts (pzsr.cn DeepGEMM page s3.1: NT, TN,
NN, TT; s3.2: grouping along K for MoE weight gradients).

* dg_transpose_fp8 is bit-exact against numpy's transpose.
* dg_fp8_gemm in every layout: within the GEMM tolerance of the oracle's
  product of the logical operands, and bit-identical to dg_fp8_gemm_nt on
  the same logical operands (the transposed copies feed the same kernels).
* dg_fp8_grouped_gemm_k: each group within tolerance of the oracle's
  K-grouped product, bit-identical to dg_fp8_gemm_nt on that group's K slice
  (same tile kernel, same K blocks in the same order), empty groups zero."""
import numpy as np
import pytest
import torch

import datagen
from gpu_util import assert_close, bf16_to_f64, dev, need_gpu, tile_points

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


@pytest.mark.parametrize("rows,cols", [(16, 16), (128, 256), (144, 400), (400, 16),
                                       (4096, 7168), (1040, 2064)])
def test_transpose_bit_exact(dg, rows, cols):
    g = np.random.default_rng(rows + cols)
    x = g.integers(0, 256, (rows, cols), dtype=np.uint8)
    out = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    dg.dg_transpose_fp8(out, dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), x.T)


def operands(orc, M, N, K, br, seed):
    qa, sa = orc.quantize(datagen.normal((M, K), 1.0, seed=seed, stream=0), br)
    qb, sb = orc.quantize(datagen.normal((N, K), 0.02, seed=seed, stream=1), 128)
    return qa, sa, qb, sb


@pytest.mark.parametrize("layout", ["nt", "tn", "nn", "tt"])
@pytest.mark.parametrize("M,N,K,br", [(256, 384, 512, 128), (300, 528, 640, 1), (48, 1040, 1024, 1),
                                      (16, 4096, 8192, 1), (1, 16384, 256, 1)])
def test_gemm_layouts(dg, orc, layout, M, N, K, br):
    if layout in ("tn", "tt") and M % 16:
        pytest.skip("A given [K][M] needs M % 16 == 0")
    qa, sa, qb, sb = operands(orc, M, N, K, br, seed=M + N + K)
    a = np.ascontiguousarray(qa.T) if layout in ("tn", "tt") else qa
    b = np.ascontiguousarray(qb.T) if layout in ("tn", "nn") else qb
    nb = dg.dg_fp8_gemm_workspace_bytes(M, N, K, layout)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm(c, dev(a), dev(b), dev(sa), dev(sb), br, layout=layout, workspace=ws)
    nt_ws = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    w2 = torch.zeros(max(nt_ws, 16), dtype=torch.uint8, device="cuda") if nt_ws else None
    c_nt = torch.empty_like(c)
    dg.dg_fp8_gemm_nt(c_nt, dev(qa), dev(qb), dev(sa), dev(sb), br, workspace=w2)
    torch.cuda.synchronize()
    assert torch.equal(c, c_nt)
    if M * N * K <= (1 << 31):
        ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=br)
        assert_close(bf16_to_f64(c), ref, what="%s %dx%dx%d" % (layout, M, N, K))


@pytest.mark.parametrize("extra", ["copies_only", "full"])
def test_gemm_layout_workspace_between_copies_and_split_k(dg, orc, extra):
    """M = 16, N = K = 4096 in the NN layout (B transposed into the
    workspace): with room for the counter region and the copy only (plus 16
    bytes, less than the split-K partials) the call runs without split-K;
    with the full size it splits K.  Both succeed, give the two-call result,
    and leave the counter region zero, so the same workspace then serves a
    split-K dg_fp8_gemm_nt call."""
    M, N, K = 16, 4096, 4096
    qa, sa, qb, sb = operands(orc, M, N, K, 1, seed=23)
    b_nn = np.ascontiguousarray(qb.T)
    full = dg.dg_fp8_gemm_workspace_bytes(M, N, K, "nn")
    nt = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    assert nt > dg.WORKSPACE_COUNTER_BYTES and full == nt + N * K
    nb = dg.WORKSPACE_COUNTER_BYTES + N * K + 16 if extra == "copies_only" else full
    ws = torch.zeros(max(nb, nt), dtype=torch.uint8, device="cuda")
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm(c, dev(qa), dev(b_nn), dev(sa), dev(sb), 1, layout="nn", workspace=ws[:nb])
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:dg.WORKSPACE_COUNTER_BYTES]) == 0
    ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1)
    assert_close(bf16_to_f64(c), ref, what="nn workspace " + extra)
    c2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm_nt(c2, dev(qa), dev(qb), dev(sa), dev(sb), 1, workspace=ws[:nt])
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:dg.WORKSPACE_COUNTER_BYTES]) == 0
    assert_close(bf16_to_f64(c2), ref, what="nt after nn")
    if extra == "full":                             # same plan: identical bits
        assert torch.equal(c.view(torch.int16), c2.view(torch.int16))


def test_gemm_layout_needs_its_workspace(dg, orc):
    qa, sa, qb, sb = operands(orc, 256, 256, 256, 128, seed=1)
    c = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dg.DGError):
        dg.dg_fp8_gemm(c, dev(qa.T.copy()), dev(qb), dev(sa), dev(sb), 128, layout="tt")


def run_k_grouped(dg, qa, sa, qb, sb, br, ko):
    M, N = qa.shape[0], qb.shape[0]
    G = len(ko) - 1
    c = torch.full((G, M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_grouped_gemm_k(c, dev(qa), dev(qb), dev(sa), dev(sb), br,
                             torch.tensor(ko, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("br", [1, 128])
def test_k_grouped_small(dg, orc, br):
    M, N, K = 300, 520, 1664
    ko = [0, 384, 384, 1024, 1152, 1664]                  # an empty group, ragged sizes
    qa, sa, qb, sb = operands(orc, M, N, K, br, seed=7)
    c = run_k_grouped(dg, qa, sa, qb, sb, br, ko)
    ref = orc.grouped_gemm_k(qa, sa, qb, sb, ko, a_block_rows=br)
    for g in range(len(ko) - 1):
        got = bf16_to_f64(c[g])
        if ko[g] == ko[g + 1]:
            assert np.all(got == 0.0)
            continue
        assert_close(got, ref[g], what="k-group %d" % g)
        k0, k1 = ko[g], ko[g + 1]
        c_nt = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        dg.dg_fp8_gemm_nt(c_nt, dev(qa[:, k0:k1]), dev(qb[:, k0:k1]),
                          dev(sa[k0 // 128:k1 // 128]), dev(sb[k0 // 128:k1 // 128]), br)
        torch.cuda.synchronize()
        assert torch.equal(c[g], c_nt), g


def test_k_grouped_weight_gradient_shape_sampled(dg, orc):
    """MoE weight-gradient shape: 8 experts, 4096 x 2048 outputs each, token
    counts 128 .. 1024 per expert (K = 4224 in all), sampled per group."""
    M, N = 4096, 2048
    sizes = [512, 128, 1024, 384, 640, 256, 896, 384]
    ko = [0]
    for s in sizes:
        ko.append(ko[-1] + s)
    K = ko[-1]
    qa, sa, qb, sb = operands(orc, M, N, K, 1, seed=11)
    c = run_k_grouped(dg, qa, sa, qb, sb, 1, ko)
    assert torch.isfinite(c).all()                  # every element written (NaN prefill)
    g_rng = np.random.default_rng(5)
    for g in range(len(sizes)):
        k0, k1 = ko[g], ko[g + 1]
        tm, tn = tile_points(M, N, 256, 256, g_rng)
        pm = np.concatenate([g_rng.integers(0, M, 600), np.full(64, M - 1), tm])
        pn = np.concatenate([g_rng.integers(0, N, 600), np.arange(0, N, N // 64), tn])
        assert pm.max() < M and pn.max() < N
        ref = orc.gemm_nt_points(np.ascontiguousarray(qa[:, k0:k1]),
                                 np.ascontiguousarray(sa[k0 // 128:k1 // 128]),
                                 np.ascontiguousarray(qb[:, k0:k1]),
                                 np.ascontiguousarray(sb[k0 // 128:k1 // 128]), pm, pn,
                                 a_block_rows=1)
        got = c[g][torch.from_numpy(pm).cuda(), torch.from_numpy(pn).cuda()]
        rms = float(np.sqrt(np.mean(ref[:600] ** 2)))
        assert_close(got.float().cpu().numpy().astype(np.float64), ref, rms=rms,
                     what="weight-gradient group %d" % g)
