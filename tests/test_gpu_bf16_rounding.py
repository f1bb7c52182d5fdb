"""BF16 rounding of the GEMM output, bit for bit, through the public entry
points (lpnh.cn FP8 block-quantised GEMM page, s4.3: FP32 accumulation,
BF16 output; the rounding is to nearest, ties to even).

Each row m of A holds one E4M3 code 1.0 (or -1.0) in its first K position
and zeros elsewhere, with its own 1x128 scale s_m; B holds code 1.0 in the
first position of every row with scale 1.  The exact product is then
+-s_m in every column, formed without rounding (1.0 * 1.0 * s_m * 1), so the
BF16 output must equal s_m rounded to BF16, which PyTorch's CPU conversion
(round to nearest even) gives.  The scales cover random finite binary32
patterns, values just below, at and above every rounding midpoint of their
BF16 neighbourhood, binary32 subnormals, and the largest finite values
(which round to infinity).  Run on the 256x256 tile kernel (many rows) and
on the small-M kernels."""
import numpy as np
import pytest
import torch

from gpu_util import need_gpu

pytestmark = pytest.mark.gpu

E4M3_ONE, E4M3_MINUS_ONE = 0x38, 0xB8


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def scale_values(n, seed):
    """n finite, non-zero binary32 bit patterns (as uint32): a quarter around
    BF16 rounding midpoints (low half 0x7FFF, 0x8000, 0x8001, 0x0000,
    0xFFFF, 0x0001 under random upper halves), then subnormals and the
    largest finite values, the rest random."""
    g = np.random.default_rng(seed)
    hi = g.integers(0, 0x7F80, n, dtype=np.uint32) << 16
    lo = np.array([0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF, 0x0001], dtype=np.uint32)
    mid = hi | lo[np.arange(n) % lo.size]
    special = np.concatenate([
        g.integers(1, 1 << 23, 64, dtype=np.uint32),                  # subnormals
        np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F7FC000,    # largest finite
                  0x00800000, 0x00000001, 0x007FFFFF, 0x00008000], dtype=np.uint32)])
    rand = g.integers(0, 1 << 31, n, dtype=np.uint32)
    pool = np.concatenate([special, mid[: max(1, n // 4)], rand])
    if n >= special.size:  # every special value, then midpoints and random ones, shuffled
        bits = pool[:n][g.permutation(n)]
    else:
        bits = pool[g.permutation(pool.size)[:n]]
    bits = bits & 0x7FFFFFFF                  # magnitudes; signs come from the codes
    exp = (bits >> 23) & 0xFF
    bits = np.where(exp == 0xFF, bits & 0x007FFFFF | 0x7F000000, bits)   # no Inf / NaN
    bits = np.where(bits == 0, np.uint32(0x3F800000), bits)              # no zero
    return bits.astype(np.uint32)


def expected_bf16(vals_f32, signs):
    t = torch.from_numpy((vals_f32 * signs).astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def run(dg, s_bits, N):
    """C = the M x N product described above; returns C's BF16 bit patterns
    and the expected ones (every column equal)."""
    M, K = s_bits.size, 128
    mag = s_bits.view(np.float32)
    # the scale is a magnitude; the sign goes into the code of odd rows
    signs = np.where(np.arange(M) % 2 == 1, -1.0, 1.0).astype(np.float32)
    a = np.zeros((M, K), dtype=np.uint8)
    a[:, 0] = np.where(signs < 0, E4M3_MINUS_ONE, E4M3_ONE)
    b = np.zeros((N, K), dtype=np.uint8)
    b[:, 0] = E4M3_ONE
    sa = mag.reshape(1, M)
    sb = np.ones((1, (N + 127) // 128), dtype=np.float32)
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    nb = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    dg.dg_fp8_gemm_nt(c, torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(),
                      torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda(), 1, workspace=ws)
    torch.cuda.synchronize()
    got = c.view(torch.int16).cpu().numpy().view(np.uint16)
    return got, expected_bf16(mag, signs)


def check(got, want, s_bits):
    bad = np.argwhere(got != want[:, None])
    assert bad.size == 0, ["in %08x: got %04x want %04x" % (s_bits[i], got[i, j], want[i])
                           for i, j in bad[:8]]


def test_bf16_rounding_tile_kernel(dg):
    s_bits = scale_values(1 << 16, seed=1)
    assert ((s_bits >> 23) == 0).sum() >= 64 and (s_bits == 0x7F7FFFFF).any()
    got, want = run(dg, s_bits, N=40)        # 256 tile rows, ragged N
    check(got, want, s_bits)


@pytest.mark.parametrize("M,N", [(1, 24), (8, 64), (16, 4096), (64, 512)])
def test_bf16_rounding_small_m_kernels(dg, M, N):
    for rep in range(4):
        s_bits = scale_values(M, seed=100 + 10 * M + rep)
        got, want = run(dg, s_bits, N)
        check(got, want, s_bits)
