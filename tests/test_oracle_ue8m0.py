"""Pins for the oracle's power-of-two (UE8M0) block scales (pzsr.cn DeepGEMM
page s3.1: UE8M0 scaling factors, four packed per 32-bit integer; the
recipe otherwise as on the lpnh.cn FP8 block-quantised GEMM page s4.2).

Reading under test: t = binary32(amax / 448) as in the FP32 recipe, the scale
is t rounded up to a power of two 2^(E - 127), E in [0, 254] (E = 0 when
t < 2^-127), codes = RNE_E4M3(binary32(x / scale)).  The exponent is checked
against math.frexp on exact Python floats, the codes against PyTorch's own
float8_e4m3fn conversion, the packing against hand-written words."""
import math

import numpy as np
import pytest
import torch

import datagen


def blocks(x, br):
    rows, cols = x.shape
    for rb in range(-(-rows // br)):
        for kb in range(-(-cols // 128)):
            yield rb, kb, x[rb * br:(rb + 1) * br, kb * 128:(kb + 1) * 128]


def expected_exponent(amax):
    t = float(np.float32(amax) / np.float32(448.0))     # binary32 division
    if t == 0.0:
        return 0
    m, ex = math.frexp(t)                                 # t = m 2^ex, m in [0.5, 1)
    e = ex - 1 if m == 0.5 else ex                        # smallest e with 2^e >= t
    return min(max(e + 127, 0), 254)


def torch_e4m3(v):
    """PyTorch's float32 -> float8_e4m3fn conversion (RNE); inputs here never
    exceed 448 by more than rounding, which it maps to 448."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("br", [128, 1])
def test_exponent_is_t_rounded_up_to_a_power_of_two(orc, br):
    g = np.random.default_rng(5)
    x = datagen.normal((256, 640), 1.0, seed=11, stream=br)
    # spread block magnitudes over a wide exponent range
    for kb in range(5):
        x[:, kb * 128:(kb + 1) * 128] *= np.float32(2.0 ** float(g.integers(-60, 60)))
    q, e = orc.quantize_ue8m0(x, br)
    for rb, kb, blk in blocks(x, br):
        amax = float(np.abs(blk).max())
        E = int(e[kb, rb])
        assert E == expected_exponent(amax), (rb, kb)
        t = float(np.float32(amax) / np.float32(448.0))
        s = math.ldexp(1.0, E - 127)
        assert s >= t and (s / 2 < t or E == 0)


@pytest.mark.parametrize("br", [128, 1])
def test_codes_match_torch_e4m3_cast_of_the_exact_quotient(orc, br):
    x = datagen.student_t_outliers(64, 1024, seed=2, stream=3)[0]
    x[:, :128] *= np.float32(1e-30)
    q, e = orc.quantize_ue8m0(x, br)
    for rb, kb, blk in blocks(x, br):
        s = np.float32(math.ldexp(1.0, int(e[kb, rb]) - 127))
        want = torch_e4m3(blk / s)                        # exact: s is a power of two
        got = q[rb * br:(rb + 1) * br, kb * 128:(kb + 1) * 128]
        assert np.array_equal(got, want), (rb, kb)


def test_power_of_two_scale_agrees_with_the_fp32_recipe(orc):
    """When amax / 448 is already a power of two, both recipes pick the same
    scale, hence the same codes."""
    x = datagen.normal((128, 512), 1.0, seed=4)
    for kb, k in enumerate([-3, 0, 5, -40]):
        blk = x[:, kb * 128:(kb + 1) * 128]
        blk /= np.abs(blk).max()
        blk *= np.float32(448.0 * 2.0 ** k)
    q8, e = orc.quantize_ue8m0(x, 128)
    q32, s32 = orc.quantize(x, 128)
    assert np.array_equal(q8, q32)
    assert np.array_equal(orc.ue8m0_scales(e), s32)


def test_one_ulp_above_a_power_of_two_takes_the_next_exponent(orc):
    x = np.zeros((1, 128), np.float32)
    amax = np.float32(448.0 * 2.0 ** -3)
    x[0, 0] = np.nextafter(amax, np.float32(np.inf))     # t just above 2^-3
    x[0, 1] = np.float32(1.0)
    q, e = orc.quantize_ue8m0(x, 1)
    assert int(e[0, 0]) == 127 - 2
    # 1.0 / 2^-2 = 4 exactly; amax / 2^-2 = 224 (1 + 2^-23) rounds to 224
    assert orc.e4m3_decode(q[0, 1]) == 4.0 and orc.e4m3_decode(q[0, 0]) == 224.0


def test_zero_tiny_and_huge_blocks(orc):
    x = np.zeros((2, 384), np.float32)
    x[0, 5] = -0.0
    x[0, 128:256] = np.float32(1e-42)                     # t far below 2^-127
    x[1, 256] = np.float32(3.0e38)                        # near the binary32 maximum
    x[1, 257] = np.float32(-1.0e38)
    x[1, 128] = np.float32(448.0 * 1.5 * 2.0 ** -127)     # t subnormal but above 2^-127
    q, e = orc.quantize_ue8m0(x, 1)
    # e is [K block][row]: zero blocks, the tiny block (row 0, K block 1)
    assert e[0, 0] == 0 and e[1, 0] == 0 and e[2, 0] == 0 and e[0, 1] == 0
    assert e[1, 1] == 1                                   # scale 2^-126 >= t > 2^-127
    assert q[0, 5] == 0x80 and q[0, 6] == 0x00
    assert int(e[2, 1]) == expected_exponent(3.0e38) and int(e[2, 1]) <= 254
    s = math.ldexp(1.0, int(e[2, 1]) - 127)
    assert abs(orc.e4m3_decode(q[1, 256]) * s - 3.0e38) <= 3.0e38 / 16
    assert orc.e4m3_decode(q[1, 257]) < 0


def test_packing_is_four_k_blocks_per_word_low_byte_first(orc):
    e = np.array([[1, 2], [3, 4], [5, 6], [7, 8], [9, 10]], np.uint8)   # 5 K blocks x 2 row blocks
    w = orc.pack_ue8m0(e).view(np.uint32)
    assert w.shape == (2, 2)
    assert w[0, 0] == 1 | 3 << 8 | 5 << 16 | 7 << 24
    assert w[0, 1] == 2 | 4 << 8 | 6 << 16 | 8 << 24
    assert w[1, 0] == 9 and w[1, 1] == 10


def test_gemm_with_power_of_two_scales_is_exact_on_integers(orc):
    """Codes for 0, +-1, +-2 and small exponents: every output is an integer
    times a power of two, computed here in Python integers."""
    g = np.random.default_rng(8)
    codes = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0], np.uint8)
    vals = np.array([0, 1, -1, 2, -2], np.int64)
    M, N, K = 4, 256, 384
    ia = g.integers(0, 5, (M, K)); ib = g.integers(0, 5, (N, K))
    ea = g.integers(124, 131, (K // 128, M)).astype(np.uint8)
    eb = g.integers(120, 135, (K // 128, N // 128)).astype(np.uint8)
    ref = orc.gemm_nt(codes[ia], orc.ue8m0_scales(ea), codes[ib], orc.ue8m0_scales(eb),
                      a_block_rows=1)
    for m in range(M):
        for n in range(0, N, 37):
            want = 0.0
            for kb in range(K // 128):
                part = int(np.sum(vals[ia[m, kb * 128:(kb + 1) * 128]] *
                                  vals[ib[n, kb * 128:(kb + 1) * 128]]))
                want += math.ldexp(part, int(ea[kb, m]) + int(eb[kb, n // 128]) - 254)
            assert ref[m, n] == want
