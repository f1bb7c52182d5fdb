"""GPU parity of the GEMM that quantises its activations itself
(dg_fp8_gemm_nt_fused_a for FP32 and dg_fp8_gemm_nt_fused_a_bf16 for BF16
activations, up to 64 rows; lpnh.cn FP8 block-quantised GEMM page, s6 on
fusing the scale computation into the GEMM, s4.2 for the quantisation).

The oracle quantises A (BF16 widened exactly to FP32 first) with 1x128
blocks and B with 128x128 blocks; its FP64 GEMM of those codes is the
reference.  Without a split-K workspace the fused result must also equal,
bit for bit, the two-call path (GPU quantiser, then dg_fp8_gemm_nt) on shapes
where that path runs the same kernel (the workgroup-staged small-M kernel:
M > 16, N >= 16384, or M > 8 with N*K above 32 Mi): any code or scale that
differed from the quantiser's would show there.  (With a workspace the two
may split K differently, so they are compared with the oracle only.)"""
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


def workspace(dg, M, N, K):
    n = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda") if n else None


def to_bf16_bits(a):
    """FP32 array -> BF16 bit patterns (round to nearest even), uint16."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def widen(a):
    """The activations as the kernel sees them before quantising: FP32, or
    BF16 bit patterns widened exactly to FP32."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a


def dev_a(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return dev(a)


def fused(dg, a, qb, sb, ws=None):
    M, N = a.shape[0], qb.shape[0]
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm_nt_fused_a(c, dev_a(a), dev(qb), dev(sb), workspace=ws)
    torch.cuda.synchronize()
    return c


def two_call(dg, a, qb, sb, ws=None):
    M, K = a.shape
    N = qb.shape[0]
    qa, sa = dg.to_fp8(dev(widen(a)), 1)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm_nt(c, qa, dev(qb), sa, dev(sb), 1, workspace=ws)
    torch.cuda.synchronize()
    return c


def same_kernel_as_two_call(M, N, K):
    """dg_fp8_gemm_nt runs the streaming kernel below these bounds; above 16
    rows both calls take the LDS-ring kernel with the same tile rows."""
    return M > 16 or not (N < 16384 and (M <= 8 or (M <= 16 and N * K <= (32 << 20))))


def weights(orc, N, K, seed):
    b = datagen.normal((N, K), 0.02, seed=seed, stream=1)
    return orc.quantize(b, 128)


def check(dg, orc, a, qb, sb, what):
    M, K = a.shape
    N = qb.shape[0]
    qa, sa = orc.quantize(widen(a), 1)
    ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1)
    ws = workspace(dg, M, N, K)
    c = fused(dg, a, qb, sb, ws)
    assert_close(bf16_to_f64(c), ref, what=what)
    assert_close(bf16_to_f64(fused(dg, a, qb, sb)), ref, what=what + " no workspace")
    if same_kernel_as_two_call(M, N, K):
        # without a workspace both run one pass over K in the same order
        assert torch.equal(fused(dg, a, qb, sb), two_call(dg, a, qb, sb)), what


@pytest.mark.parametrize("M", [1, 2, 5, 8, 13, 16])
@pytest.mark.parametrize("N,K", [(256, 512), (8, 128), (24, 256), (1000, 640), (520, 2048),
                                 (4096, 1536)])
def test_fused_full_compare(dg, orc, M, N, K):
    """Ragged N (8, 24, 520, 1000 are not multiples of the 16-row strip or the
    128-row scale block), one K block, and K splits that do not divide evenly."""
    a = datagen.normal((M, K), 1.0, seed=M * 31 + K, stream=0)
    qb, sb = weights(orc, N, K, seed=N + K)
    check(dg, orc, a, qb, sb, "fused %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(1, 16384, 256), (5, 16392, 384), (16, 2056, 16384),
                                   (11, 4104, 8320), (16, 16384, 1024)])
def test_fused_bit_equal_to_quantise_then_gemm(dg, orc, M, N, K):
    """Shapes where the two-call path runs the same small-M kernel: identical
    bits without the split-K workspace, the oracle's tolerance with it."""
    assert same_kernel_as_two_call(M, N, K)
    a = datagen.normal((M, K), 1.0, seed=M + N, stream=0)
    qb, sb = weights(orc, N, K, seed=K)
    check(dg, orc, a, qb, sb, "fused bit-equal %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [17, 33, 40, 64])
@pytest.mark.parametrize("N,K", [(256, 512), (1000, 640), (520, 2048), (4096, 1536),
                                 (24, 4096)])
def test_fused_wide_full_compare(dg, orc, M, N, K, dtype):
    """17 to 64 rows of FP32 or BF16 activations (32- and 64-row staged
    blocks, rows past M clamped), ragged N, uneven K splits: against the
    oracle with and without the split-K workspace, and bit for bit against
    the quantiser followed by dg_fp8_gemm_nt without it."""
    a = datagen.normal((M, K), 1.0, seed=M * 7 + N, stream=0)
    if dtype == "bf16":
        a = to_bf16_bits(a)
    qb, sb = weights(orc, N, K, seed=N + K)
    check(dg, orc, a, qb, sb, "fused %s %dx%dx%d" % (dtype, M, N, K))


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("N,K", [(256, 512), (520, 2048), (16384, 1024)])
def test_fused_bf16_small_batches(dg, orc, M, N, K):
    a = to_bf16_bits(datagen.normal((M, K), 1.0, seed=M + 3 * N, stream=0))
    qb, sb = weights(orc, N, K, seed=K)
    check(dg, orc, a, qb, sb, "fused bf16 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [8, 64])
def test_fused_special_blocks(dg, orc, M, dtype):
    """Blocks the quantiser treats specially [lpnh.cn page s5.4]: all zero
    (signed zeros), tiny values whose scale is a binary32 subnormal, a single
    large outlier, and a block of one repeated negative value."""
    N, K = 16384, 1024
    a = datagen.normal((M, K), 1.0, seed=5, stream=0)
    a[0, 128:256] = 0.0
    a[0, 130] = -0.0
    # values whose block scale amax / 448 is a binary32 subnormal (BF16 keeps
    # subnormals down to 2^-133, so its block uses larger ones)
    a[1, 0:128] = datagen.normal((1, 128), 1e-41 if dtype == "f32" else 4e-39, seed=6,
                                 stream=0)[0]
    a[2, 300] = 3.0e4
    a[3, 512:640] = -2.5
    a[7, :] = 0.0
    a = a.astype(np.float32)
    if dtype == "bf16":
        a = to_bf16_bits(a)
        assert 0 < np.abs(widen(a)[1, :128]).max() / np.float32(448) < np.float32(2.0 ** -126)
    qb, sb = weights(orc, N, K, seed=9)
    check(dg, orc, a, qb, sb, "fused special blocks %d %s" % (M, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 16, 64])
@pytest.mark.parametrize("N,K", [(24576, 1536), (7168, 16384), (4096, 4096)])
def test_fused_decode_shapes_sampled(dg, orc, M, N, K, dtype):
    """The decode shapes at full size, compared on sampled elements (whole rows
    and columns plus random points)."""
    a = datagen.normal((M, K), 1.0, seed=M, stream=0)
    if dtype == "bf16":
        a = to_bf16_bits(a)
    qb, sb = weights(orc, N, K, seed=N)
    qa, sa = orc.quantize(widen(a), 1)
    ws = workspace(dg, M, N, K)
    c = fused(dg, a, qb, sb, ws)
    assert torch.isfinite(c).all()                  # every element written (NaN prefill)
    g = np.random.default_rng(N)
    tm, tn = tile_points(M, N, 64, 64, g)
    pm = np.concatenate([g.integers(0, M, 1500), np.full(N, M - 1),
                         np.arange(M), np.arange(M), tm])
    pn = np.concatenate([g.integers(0, N, 1500), np.arange(N),
                         np.zeros(M, dtype=np.int64), np.full(M, N - 1), tn])
    assert pm.max() < M and pn.max() < N
    ref = orc.gemm_nt_points(qa, sa, qb, sb, pm, pn, a_block_rows=1)
    got = c[torch.from_numpy(pm).cuda(), torch.from_numpy(pn).cuda()]
    rms = float(np.sqrt(np.mean(ref[:1500] ** 2)))
    assert_close(got.float().cpu().numpy().astype(np.float64), ref, rms=rms,
                 what="fused decode %s %dx%dx%d" % (dtype, M, N, K))
    if same_kernel_as_two_call(M, N, K):
        assert torch.equal(fused(dg, a, qb, sb), two_call(dg, a, qb, sb))


def test_fused_deterministic(dg, orc):
    M, N, K = 16, 4096, 4096
    a = datagen.normal((M, K), 1.0, seed=3, stream=0)
    qb, sb = weights(orc, N, K, seed=4)
    ws = workspace(dg, M, N, K)
    c1, c2 = fused(dg, a, qb, sb, ws), fused(dg, a, qb, sb, ws)
    assert torch.equal(c1, c2)


def test_fused_rejects_large_batches(dg):
    a = torch.zeros((dg.FUSED_A_MAX_M + 1, 128), dtype=torch.float32, device="cuda")
    b = torch.zeros((256, 128), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((1, 2), dtype=torch.float32, device="cuda")
    c = torch.empty((a.shape[0], 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dg.DGError):
        dg.dg_fp8_gemm_nt_fused_a(c, a, b, sb)
