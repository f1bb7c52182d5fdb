"""Pins for the oracle's block quantiser (lpnh.cn page on the FP8
block-quantised GEMM: s3.1 scale = max_abs/448 in FP32, s4.2 recipe, s5.4
all-zero blocks), checked against exact-rational brute force, closed forms
and invariants -- never against the oracle itself."""
import json
import os

import numpy as np
import pytest

import datagen
import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex32(a):
    return [hex(int(v)) for v in np.asarray(a, dtype=np.float32).view(np.uint32).ravel()]


def test_hand_4x4_codes_and_scales(orc):
    with open(os.path.join(GOLDEN, "hand_4x4.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], dtype=np.float32)
    B = np.array(g["B"], dtype=np.float32)
    blk = g["block_128x128"]
    qa, sa = orc.quantize(A, 128)
    qb, sb = orc.quantize(B, 128)
    assert _hex32(sa) == blk["sA_hex"] and _hex32(sb) == blk["sB_hex"]
    assert ["%02X" % c for c in qa.ravel()] == blk["qA_hex"]
    assert ["%02X" % c for c in qb.ravel()] == blk["qB_hex"]
    # the fixture itself re-derived by exact brute force
    eqa, esa = exact.quantize_exact(A, 128)
    assert np.array_equal(eqa, qa) and np.array_equal(esa, sa)
    row = g["a_block_1x128"]
    qa1, sa1 = orc.quantize(A, 1)
    assert _hex32(sa1) == row["sA_hex"]
    assert ["%02X" % c for c in qa1.ravel()] == row["qA_hex"]
    eqa1, esa1 = exact.quantize_exact(A, 1)
    assert np.array_equal(eqa1, qa1) and np.array_equal(esa1, sa1)


@pytest.mark.parametrize("rows,cols,block_rows", [
    (3, 130, 1), (5, 256, 128), (130, 20, 128), (2, 300, 128), (4, 129, 1)])
def test_quantize_matches_exact_bruteforce(orc, rows, cols, block_rows):
    x = datagen.normal((rows, cols), 1.0, seed=rows * 1000 + cols, stream=3)
    x[0, 0] = -0.0
    x[-1, -1] = np.float32(1e-30)
    q, s = orc.quantize(x, block_rows)
    eq, es = exact.quantize_exact(x, block_rows)
    assert np.array_equal(s.view(np.uint32), es.view(np.uint32))
    assert np.array_equal(q, eq)


def test_amax_element_maps_to_448_and_scale_is_fp32_division(orc):
    x = datagen.normal((256, 384), 0.02, seed=5, stream=1)
    for br in (1, 128):
        q, s = orc.quantize(x, br)
        n_rb = s.shape[1]
        for kb in range(s.shape[0]):
            for rb in range(n_rb):
                blk = x[rb * br:(rb + 1) * br, kb * 128:(kb + 1) * 128]
                qb = q[rb * br:(rb + 1) * br, kb * 128:(kb + 1) * 128]
                amax = np.abs(blk).max()
                # scale bits equal binary32(amax/448) whether formed in FP32 or FP64
                assert s[kb, rb] == np.float32(amax) / np.float32(448.0)
                assert s[kb, rb] == np.float32(np.float64(amax) / 448.0)
                i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                assert (qb[i] & 0x7F) == 0x7E
                assert (qb[i] >> 7) == (1 if blk[i] < 0 else 0)
                assert np.all((qb & 0x7F) <= 0x7E)      # never NaN


def test_all_zero_block_has_zero_scale_and_signed_zero_codes(orc):
    x = datagen.normal((4, 256), 1.0, seed=9)
    x[:, :128] = 0.0
    x[1, 5] = -0.0
    q, s = orc.quantize(x, 128)
    assert s[0, 0] == 0.0 and s[1, 0] > 0
    assert q[1, 5] == 0x80 and np.count_nonzero(q[:, :128]) == 1


def test_quantisation_error_bound(orc):
    x = datagen.normal((256, 512), 1.0, seed=11)
    x[:, 7] *= np.float32(1e-4)       # push some elements into the subnormal grid
    q, s = orc.quantize(x, 128)
    d = exact.torch_decode(q)
    srep = np.repeat(np.repeat(s.T, 128, axis=0), 128, axis=1)[:256, :512].astype(np.float64)
    v = x.astype(np.float64) / srep
    err = np.abs(v - d)
    normal = np.abs(d) >= 2.0 ** -6
    # half an ulp of a 3-bit significand, plus the binary32 quotient rounding
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(v[normal]) * (1 + 2.0 ** -20))
    assert np.all(err[~normal] <= 2.0 ** -10 * (1 + 2.0 ** -20))


def test_power_of_two_scaling_identity(orc):
    x = datagen.normal((130, 300), 1.0, seed=13)
    q, s = orc.quantize(x, 128)
    for j in (-20, -3, 5, 30):
        q2, s2 = orc.quantize(x * np.float32(2.0 ** j), 128)
        assert np.array_equal(q2, q)
        assert np.array_equal(s2, s * np.float32(2.0 ** j))


def test_row_blocks_equal_tile_blocks_when_rows_share_amax(orc):
    x = datagen.normal((128, 256), 1.0, seed=17)
    for kb in range(2):
        sl = slice(kb * 128, (kb + 1) * 128)
        amax = np.abs(x[:, sl]).max()
        x[:, kb * 128 + 3] = amax        # every row of the group holds the block amax
    q1, s1 = orc.quantize(x, 1)
    q128, s128 = orc.quantize(x, 128)
    assert np.array_equal(q1, q128)
    assert np.all(s1 == s128[:, :1])


def test_clipped_edge_blocks_equal_zero_padding(orc):
    x = datagen.normal((200, 333), 1.0, seed=19)
    xp = np.zeros((256, 384), dtype=np.float32)
    xp[:200, :333] = x
    for br in (1, 128):
        q, s = orc.quantize(x, br)
        qp, sp = orc.quantize(xp, br)
        assert np.array_equal(qp[:200, :333], q)
        assert np.array_equal(sp[:, :s.shape[1]], s)


def test_global_scale_equals_single_block_and_bruteforce(orc):
    """Per-tensor scaling (bjdmk.com.cn page s3.3 contrasts it with per-block
    scales): for a tensor that is one 128x128 block it is the block quantiser;
    for a larger tensor it is the same rounding with s = amax(tensor)/448,
    checked element by element against the exact-rational nearest-even search."""
    x = datagen.normal((100, 128), 1.0, seed=21, stream=1)
    qg, sg = orc.quantize_global(x)
    qb, sb = orc.quantize(x, 128)
    assert sb.shape == (1, 1) and np.float32(sg).view(np.uint32) == sb[0, 0].view(np.uint32)
    assert np.array_equal(qg, qb)

    y = datagen.normal((5, 300), 1.0, seed=22, stream=1)
    y[2, 7] = np.float32(37.5)          # one large element sets the tensor scale
    y[0, 0] = -0.0
    qg, sg = orc.quantize_global(y)
    amax = max(abs(float(v)) for v in y.ravel())
    assert np.float32(sg) == np.float32(amax) / np.float32(448.0)
    for (i, j), v in np.ndenumerate(y):
        want = exact.nearest_even_code(exact.Fraction(float(np.float32(v) / np.float32(sg))),
                                       bool(np.signbit(v)))
        assert qg[i, j] == want, (i, j)
    assert qg[2, 7] == 0x7E             # the amax element lands on 448


def test_global_scale_power_of_two_invariance_and_zero(orc):
    x = datagen.normal((7, 260), 3.0, seed=23, stream=1)
    q1, s1 = orc.quantize_global(x)
    q2, s2 = orc.quantize_global(x * np.float32(2.0 ** -12))
    assert np.array_equal(q1, q2) and s2 == s1 * 2.0 ** -12
    z = np.zeros((3, 16), np.float32)
    z[1, 2] = -0.0
    qz, sz = orc.quantize_global(z)
    assert sz == 0.0 and qz[1, 2] == 0x80 and int(qz.sum()) == 0x80


def test_block_scaling_beats_global_on_outlier_activations(orc):
    """The point of fine-grained scales: with heavy-tailed rows and a few
    outlier channels, one tensor-wide scale is set by the largest element of
    the whole tensor and pushes the other rows' values down to the coarse
    (subnormal) end of E4M3; per-row 128-wide blocks adapt to each row.
    Relative Frobenius error of the dequantised tensor (seeded input)."""
    x, hot = datagen.student_t_outliers(64, 1024, seed=0, stream=5)
    qb, sb = orc.quantize(x, 1)
    qg, sg = orc.quantize_global(x)
    dec = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    xb = dec[qb] * np.repeat(sb.T, 128, axis=1)[:, :1024]
    xg = dec[qg] * sg
    err_b = np.linalg.norm(xb - x) / np.linalg.norm(x)
    err_g = np.linalg.norm(xg - x) / np.linalg.norm(x)
    assert len(hot) == 10
    assert err_b < 0.5 * err_g
