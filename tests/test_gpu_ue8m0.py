"""GPU parity of the power-of-two (UE8M0) scale path (pzsr.cn DeepGEMM page
s3.1; the recipe otherwise as on the lpnh.cn FP8 block-quantised GEMM page
s4.2): the quantiser's codes and packed exponent words must equal the
oracle's bit for bit; the GEMM, which applies the scales inside gfx950's
scaled FP8 matrix instruction, must meet the GEMM tolerance against the
oracle's FP64 product of the same codes and scales."""
import numpy as np
import pytest
import torch

import datagen
from gpu_util import assert_close, bf16_to_f64, dev, need_gpu, oracle_gemm_rows, tile_points

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def gpu_quant(dg, x, br):
    q, sf = dg.to_fp8_ue8m0(dev(x), br)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


def check_quant(dg, orc, x, br, what):
    q, sf = gpu_quant(dg, x, br)
    oq, oe = orc.quantize_ue8m0(x, br)
    assert np.array_equal(q, oq), what
    assert np.array_equal(sf, orc.pack_ue8m0(oe)), what


@pytest.mark.parametrize("br", [128, 1])
@pytest.mark.parametrize("rows,cols", [(128, 512), (256, 640), (1, 128), (3, 16), (200, 384),
                                       (129, 1024), (300, 144), (64, 1664)])
def test_quantize_ue8m0_small_and_ragged(dg, orc, rows, cols, br):
    """Ragged rows and columns, K-block counts of 1 to 13 (partial last words)."""
    x = datagen.normal((rows, cols), 1.0, seed=rows + cols, stream=br)
    check_quant(dg, orc, x, br, "%dx%d/%d" % (rows, cols, br))


@pytest.mark.parametrize("br", [128, 1])
def test_quantize_ue8m0_special_blocks(dg, orc, br):
    x = datagen.normal((256, 1024), 0.02, seed=3)
    x[:128, :128] = 0.0
    x[5, 7] = -0.0
    x[:, 128:256] *= np.float32(1e-38)                   # t subnormal
    x[:, 256:384] *= np.float32(1e-44)                   # t below 2^-127: E = 0
    x[:, 384:512] = np.float32(2.0) ** np.arange(-20, 108, dtype=np.float32)[None, :]
    x[:, 512:640] *= np.float32(1e30)
    blk = x[:, 640:768]
    blk /= np.abs(blk).max()
    blk *= np.float32(448.0 * 2.0 ** -5)                 # t exactly a power of two
    x[0, 768] = np.nextafter(np.float32(448.0), np.float32(np.inf))   # t one ulp above 1
    x[3, 896:] = -np.abs(x[3, 896:])
    check_quant(dg, orc, x, br, "special/%d" % br)


@pytest.mark.parametrize("rows,cols,br", [(4096, 7168, 128), (64, 16384, 1), (2816, 11008, 1)])
def test_quantize_ue8m0_full_size(dg, orc, rows, cols, br):
    x = datagen.normal((rows, cols), 1.0 if br == 1 else 0.02, seed=0, stream=1)
    check_quant(dg, orc, x, br, "%dx%d/%d" % (rows, cols, br))


def operands(orc, M, N, K, br, seed=0):
    a = datagen.normal((M, K), 1.0, seed=seed, stream=0)
    b = datagen.normal((N, K), 0.02, seed=seed, stream=1)
    qa, ea = orc.quantize_ue8m0(a, br)
    qb, eb = orc.quantize_ue8m0(b, 128)
    return qa, ea, qb, eb


def run_gemm(dg, orc, qa, ea, qb, eb, br):
    M, N = qa.shape[0], qb.shape[0]
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm_nt_ue8m0(c, dev(qa), dev(qb), dev(orc.pack_ue8m0(ea)),
                            dev(orc.pack_ue8m0(eb)), br)
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("br", [128, 1])
@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (256, 256, 128), (512, 768, 384),
                                   (300, 520, 1024), (200, 264, 640), (1, 256, 256),
                                   (16, 512, 1664), (257, 136, 128),
                                   # tile order of the full-size launches: > 4 tile rows,
                                   # >= 8 tiles, ragged
                                   (1300, 2312, 256), (2100, 1800, 384)])
def test_gemm_ue8m0_small_full_compare(dg, orc, M, N, K, br):
    """Several tiles, ragged M and N, K-block counts that leave partial words."""
    qa, ea, qb, eb = operands(orc, M, N, K, br, seed=M + N + K)
    ref = oracle_gemm_rows(orc, qa, orc.ue8m0_scales(ea), qb, orc.ue8m0_scales(eb), br)
    c = bf16_to_f64(run_gemm(dg, orc, qa, ea, qb, eb, br))
    assert_close(c, ref, what="ue8m0 %dx%dx%d/%d" % (M, N, K, br))


def test_gemm_ue8m0_exact_on_integers(dg, orc):
    """Codes for 0, +-1, +-2 with exponents that vary per row (A) and per
    128-row block (B): every output is a small integer times a power of two
    that BF16 holds exactly, so the result must be bit-exact.  Pins which
    exponent byte applies to which row and column."""
    g = np.random.default_rng(9)
    codes = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0], np.uint8)
    M, N, K = 256, 512, 640
    qa = codes[g.integers(0, 5, (M, K))]
    qb = codes[g.integers(0, 5, (N, K))]
    qa[:, 2:] = 0                # one K block with two products per output: |sum| <= 8,
                                 # times one power of two -- exact in BF16
    ea = g.integers(124, 131, (K // 128, M)).astype(np.uint8)
    eb = g.integers(122, 133, (K // 128, N // 128)).astype(np.uint8)
    ref = orc.gemm_nt(qa, orc.ue8m0_scales(ea), qb, orc.ue8m0_scales(eb), a_block_rows=1)
    c = bf16_to_f64(run_gemm(dg, orc, qa, ea, qb, eb, 1))
    assert np.array_equal(c, ref)


def test_gemm_ue8m0_one_hot_exponents(dg, orc):
    """All codes 1.0; one A row, one B row block and one K block at a time get
    a larger exponent: exactly the outputs that block feeds must change."""
    M, N, K = 256, 512, 512
    qa = np.full((M, K), 0x38, np.uint8)
    qb = np.full((N, K), 0x38, np.uint8)
    base_a = np.full((K // 128, M), 127, np.uint8)
    base_b = np.full((K // 128, N // 128), 127, np.uint8)
    for (kb, m, nb) in [(0, 0, 0), (3, 200, 1), (1, 17, 3), (2, 255, 2)]:
        ea = base_a.copy(); ea[kb, m] = 130
        eb = base_b.copy(); eb[kb, nb] = 125
        ref = orc.gemm_nt(qa, orc.ue8m0_scales(ea), qb, orc.ue8m0_scales(eb), a_block_rows=1)
        c = bf16_to_f64(run_gemm(dg, orc, qa, ea, qb, eb, 1))
        assert np.array_equal(c, ref), (kb, m, nb)


def test_gemm_ue8m0_full_size_sampled(dg, orc):
    M, N, K, br = 4096, 4096, 7168, 128
    qa, ea, qb, eb = operands(orc, M, N, K, br)
    c = run_gemm(dg, orc, qa, ea, qb, eb, br)
    assert torch.isfinite(c).all()                  # every element written (NaN prefill)
    g = np.random.default_rng(1)
    tm, tn = tile_points(M, N, 256, 256, g)
    pm = np.concatenate([g.integers(0, M, 1500), np.full(N, M - 1), np.arange(0, M, 8), tm])
    pn = np.concatenate([g.integers(0, N, 1500), np.arange(N), np.full(M // 8, N - 1), tn])
    assert pm.max() < M and pn.max() < N
    ref = orc.gemm_nt_points(qa, orc.ue8m0_scales(ea), qb, orc.ue8m0_scales(eb), pm, pn,
                             a_block_rows=br)
    got = c[torch.from_numpy(pm).cuda(), torch.from_numpy(pn).cuda()]
    rms = float(np.sqrt(np.mean(ref[:1500] ** 2)))
    assert_close(got.float().cpu().numpy().astype(np.float64), ref, rms=rms,
                 what="ue8m0 %dx%dx%d" % (M, N, K))


def test_end_to_end_ue8m0_and_determinism(dg, orc):
    """GPU quantiser feeding the GPU GEMM, against the oracle on the same FP32
    inputs; two runs give identical bits."""
    M, N, K = 512, 768, 1024
    a = datagen.normal((M, K), 1.0, seed=21, stream=0)
    b = datagen.normal((N, K), 0.02, seed=21, stream=1)
    qa, sfa = dg.to_fp8_ue8m0(dev(a), 1)
    qb, sfb = dg.to_fp8_ue8m0(dev(b), 128)
    outs = []
    for _ in range(2):
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        dg.dg_fp8_gemm_nt_ue8m0(c, qa, qb, sfa, sfb, 1)
        outs.append(c)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    oqa, oea = orc.quantize_ue8m0(a, 1)
    oqb, oeb = orc.quantize_ue8m0(b, 128)
    ref = orc.gemm_nt(oqa, orc.ue8m0_scales(oea), oqb, orc.ue8m0_scales(oeb), a_block_rows=1)
    assert_close(bf16_to_f64(outs[0]), ref, what="ue8m0 end to end")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 512), (5, 2056, 1024), (16, 136, 2048), (33, 1000, 640),
                                   (64, 384, 4096), (2, 24576, 384), (16, 2056, 16384),
                                   (12, 16392, 384)])
@pytest.mark.parametrize("use_ws", [False, True])
def test_gemm_ue8m0_small_m(dg, orc, M, N, K, use_ws):
    """The small-M kernels with power-of-two scales (the streaming kernel, the
    LDS-ring kernel with and without split-K), ragged N, K ranges that split
    unevenly: compared with the oracle in full."""
    qa, ea, qb, eb = operands(orc, M, N, K, 1, seed=M * 5 + N)
    ws = None
    if use_ws:
        nb = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
        ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm_nt_ue8m0(c, dev(qa), dev(qb), dev(orc.pack_ue8m0(ea)), dev(orc.pack_ue8m0(eb)),
                            1, workspace=ws)
    torch.cuda.synchronize()
    ref = orc.gemm_nt(qa, orc.ue8m0_scales(ea), qb, orc.ue8m0_scales(eb), a_block_rows=1)
    assert_close(bf16_to_f64(c), ref, what="ue8m0 small-M %dx%dx%d ws=%s" % (M, N, K, use_ws))


def test_gemm_ue8m0_small_m_extreme_exponents(dg, orc):
    """Exponent bytes near both ends of the range on the small-M paths: the K
    steps past a split's range must add nothing even where 2^(Ea+Eb-254)
    is large (they zero an operand, as UE8M0 has no zero scale)."""
    for (M, N, K) in [(4, 1032, 1280), (16, 4104, 8320), (40, 1032, 640)]:
        g = np.random.default_rng(M + N)
        codes = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0], np.uint8)
        qa = codes[g.integers(0, 5, (M, K))]
        qb = codes[g.integers(0, 5, (N, K))]
        ea = g.integers(150, 160, (K // 128, M)).astype(np.uint8)
        eb = g.integers(100, 110, (K // 128, -(-N // 128))).astype(np.uint8)
        for use_ws in (False, True):
            ws = None
            if use_ws:
                nb = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
                ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda")
            c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            dg.dg_fp8_gemm_nt_ue8m0(c, dev(qa), dev(qb), dev(orc.pack_ue8m0(ea)),
                                    dev(orc.pack_ue8m0(eb)), 1, workspace=ws)
            torch.cuda.synchronize()
            ref = orc.gemm_nt(qa, orc.ue8m0_scales(ea), qb, orc.ue8m0_scales(eb), a_block_rows=1)
            assert_close(bf16_to_f64(c), ref, what="ue8m0 extreme %dx%dx%d" % (M, N, K))


def grouped_ue8m0_operands(orc, tokens, G, N, K, br, seed):
    r = datagen.moe_routing(tokens, G, min(2, G), align=128, seed=seed)
    mi = r["m_indices"]
    a = datagen.gather_rows(datagen.normal((tokens, K), 1.0, seed=seed, stream=1), r["row_token"])
    qa, ea = orc.quantize_ue8m0(a, br)
    w = datagen.normal((G * N, K), 0.02, seed=seed, stream=2)
    qb = np.empty((G, N, K), np.uint8)
    ebs = []
    for e in range(G):
        qb[e], eb = orc.quantize_ue8m0(w[e * N:(e + 1) * N], 128)
        ebs.append(eb)
    return qa, ea, qb, ebs, mi


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("tokens,G,N,K", [(100, 3, 264, 640), (300, 4, 512, 1152), (64, 8, 136, 128)])
def test_grouped_gemm_ue8m0(dg, orc, tokens, G, N, K, br):
    """Grouped M-contiguous GEMM with UE8M0 scales (pzsr.cn DeepGEMM page
    s3.1, s3.2): against the oracle's grouped FP64 product with the
    exponents as FP32 powers of two; padding rows exact zeros; K-block counts
    that leave partial exponent words."""
    qa, ea, qb, ebs, mi = grouped_ue8m0_operands(orc, tokens, G, N, K, br, seed=tokens + G)
    M = qa.shape[0]
    sfb = np.stack([orc.pack_ue8m0(eb) for eb in ebs])
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_grouped_gemm_contig_ue8m0(c, dev(qa), dev(qb), dev(orc.pack_ue8m0(ea)), dev(sfb), br,
                                        dev(mi))
    torch.cuda.synchronize()
    got = bf16_to_f64(c)
    real = mi >= 0
    assert np.all(got[~real] == 0.0)
    sb = np.stack([orc.ue8m0_scales(eb) for eb in ebs])
    ref = orc.grouped_gemm_contig(qa, orc.ue8m0_scales(ea), qb, sb, mi, a_block_rows=br)
    assert_close(got[real], ref[real], what="grouped ue8m0 %d/%d/%d/%d/%d" % (tokens, G, N, K, br))


def test_grouped_gemm_ue8m0_one_expert_equals_dense(dg, orc):
    qa, ea, qb, ebs, mi = grouped_ue8m0_operands(orc, 256, 1, 512, 1024, 1, seed=41)
    M, N = qa.shape[0], qb.shape[1]
    sfa = dev(orc.pack_ue8m0(ea))
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_grouped_gemm_contig_ue8m0(c, dev(qa), dev(qb), sfa,
                                        dev(orc.pack_ue8m0(ebs[0])[None]), 1, dev(mi))
    cd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm_nt_ue8m0(cd, dev(qa), dev(qb[0]), sfa, dev(orc.pack_ue8m0(ebs[0])), 1)
    torch.cuda.synchronize()
    real = mi >= 0
    assert np.array_equal(bf16_to_f64(c)[real], bf16_to_f64(cd)[real])


MASKED_UE8M0_CASES = [
    # G, max_m, N, K, br, masks
    (6, 40, 1024, 4224, 1, [40, 0, 9, 33, 1, 17]),
    (6, 40, 1024, 4224, 128, [40, 0, 9, 33, 1, 17]),
    (3, 100, 256, 4224, 1, [100, 64, 65]),        # two 64-row chunks: row offset 64
    (2, 200, 256, 4224, 128, [200, 130]),         # four chunks, second 128-row scale block
]


@pytest.mark.parametrize("ws", [False, True])
@pytest.mark.parametrize("G,max_m,N,K,br,mm", MASKED_UE8M0_CASES)
def test_masked_grouped_gemm_ue8m0(dg, orc, G, max_m, N, K, br, mm, ws):
    """Masked grouped layout with UE8M0 scales: valid rows within the GEMM
    tolerance of the oracle's masked product (exponents as FP32 powers of
    two), rows past the counts untouched; K-block counts leaving partial
    exponent words; several row chunks per group (A rows and exponent words
    offset per chunk); with and without the split-K workspace."""
    mm = np.array(mm, np.int32)
    qa = np.empty((G, max_m, K), np.uint8)
    qb = np.empty((G, N, K), np.uint8)
    eas, ebs = [], []
    for g in range(G):
        qa[g], ea = orc.quantize_ue8m0(datagen.normal((max_m, K), 1.0, seed=g, stream=5), br)
        qb[g], eb = orc.quantize_ue8m0(datagen.normal((N, K), 0.02, seed=g, stream=6), 128)
        eas.append(ea)
        ebs.append(eb)
    sfa = np.stack([orc.pack_ue8m0(e) for e in eas])
    sfb = np.stack([orc.pack_ue8m0(e) for e in ebs])
    c = torch.full((G, max_m, N), 0x4B1D, dtype=torch.int16, device="cuda")
    w = None
    if ws:
        nb = dg.dg_fp8_grouped_gemm_masked_workspace_bytes(G, max_m, N, K)
        assert nb > 0
        w = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    dg.dg_fp8_grouped_gemm_masked_ue8m0(c, dev(qa), dev(qb), dev(sfa), dev(sfb), br, dev(mm),
                                        workspace=w)
    torch.cuda.synchronize()
    bits = c.cpu().numpy().view(np.uint16)
    got = bf16_to_f64(c)
    sa = np.stack([orc.ue8m0_scales(e) for e in eas])
    sb = np.stack([orc.ue8m0_scales(e) for e in ebs])
    ref = orc.grouped_gemm_masked(qa, sa, qb, sb, mm, a_block_rows=br)
    valid = ~np.isnan(ref)
    assert np.all(bits[~valid] == 0x4B1D)
    assert_close(got[valid], ref[valid], what="masked ue8m0 br=%d ws=%s" % (br, ws))
