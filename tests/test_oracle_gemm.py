"""Pins for the oracle's dequantised NT GEMM and grouped GEMM.

C[m,n] = sum_kb sa*sb*sum_{k in kb} dec(a[m,k]) dec(b[n,k]) (lpnh.cn page on the
FP8 block-quantised GEMM, s2.2 and s3.2; NT layout from the pzsr.cn DeepGEMM
page, s3.1 and s4.1; grouped contiguous layout, same page s3.2 and s3.3).
Independent checks: exact rationals on tiny shapes, numpy float64 matmul of
PyTorch-decoded operands, integer matmul for the exactness probe, one-hot
probes, the hand 4x4 case, and power-of-two scale identities.
"""
import json
import os

import numpy as np
import pytest

import datagen
import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_codes(g, shape):
    c = g.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E          # no NaN codes
    return c


def _rand_scales(g, shape):
    return (g.random(shape) * 0.01 + 1e-4).astype(np.float32)


def _dequant_matmul(qa, sa, qb, sb, a_block_rows):
    """float64 numpy reference: expand scales onto the elements, decode with
    torch, and call matmul."""
    da = exact.torch_decode(qa)
    db = exact.torch_decode(qb)
    M, K = da.shape
    N = db.shape[0]
    kb = np.arange(K) // 128
    sa_el = sa.astype(np.float64)[kb[None, :], (np.arange(M) // a_block_rows)[:, None]]
    sb_el = sb.astype(np.float64)[kb[None, :], (np.arange(N) // 128)[:, None]]
    return (da * sa_el) @ (db * sb_el).T


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 5, 128), (5, 2, 256), (4, 4, 200)])
@pytest.mark.parametrize("br", [1, 128])
def test_gemm_matches_exact_rationals(orc, M, N, K, br):
    g = np.random.default_rng(M * 100 + N * 10 + K + br)
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (N, K))
    sa = _rand_scales(g, (-(-K // 128), -(-M // br)))
    sb = _rand_scales(g, (-(-K // 128), -(-N // 128)))
    ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=br)
    ex = exact.gemm_exact(qa, sa, qb, sb, br)
    n_kb = -(-K // 128)
    for m in range(M):
        for n in range(N):
            e = float(ex[m][n])
            # each block sum is exact; only the n_kb scaled additions round
            bound = n_kb * 2.0 ** -52 * sum(
                abs(float(sa[kb, m // br]) * float(sb[kb, n // 128])) * 448.0 * 448.0 * 128
                for kb in range(n_kb))
            assert abs(ref[m, n] - e) <= bound


@pytest.mark.parametrize("br", [1, 128])
def test_gemm_matches_float64_matmul(orc, br):
    M, N, K = 150, 260, 384
    a = datagen.normal((M, K), 1.0, seed=21, stream=0)
    b = datagen.normal((N, K), 0.02, seed=21, stream=1)
    qa, sa = orc.quantize(a, br)
    qb, sb = orc.quantize(b, 128)
    ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=br)
    mm = _dequant_matmul(qa, sa, qb, sb, br)
    rms = np.sqrt(np.mean(mm ** 2))
    assert np.max(np.abs(ref - mm)) <= 1e-12 * rms
    # and the quantised product is close to the unquantised one
    full = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.linalg.norm(ref - full) / np.linalg.norm(full) < 0.05


def test_exactness_probe_unit_scales_small_integer_codes(orc):
    """Unit scales and codes for 0, +-1, +-2 (the lpnh.cn page, s6, suggests
    scales of 1.0 and values exact in FP8): every result is an exact integer."""
    g = np.random.default_rng(3)
    codes = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0], dtype=np.uint8)   # 0, 1, -1, 2, -2
    vals = np.array([0, 1, -1, 2, -2], dtype=np.int64)
    ia = g.integers(0, 5, size=(64, 128))
    ib = g.integers(0, 5, size=(96, 128))
    ref = orc.gemm_nt(codes[ia], np.ones((1, 1), np.float32), codes[ib],
                      np.ones((1, 1), np.float32), a_block_rows=128)
    assert np.array_equal(ref, (vals[ia] @ vals[ib].T).astype(np.float64))


def test_one_hot_probes(orc):
    g = np.random.default_rng(4)
    M, N, K = 6, 200, 256
    qb = _rand_codes(g, (N, K))
    sb = _rand_scales(g, (2, 2))
    sa = _rand_scales(g, (2, 6))
    db = exact.torch_decode(qb)
    for (m, k) in [(0, 0), (5, 255), (3, 130)]:
        qa = np.zeros((M, K), dtype=np.uint8)
        qa[m, k] = 0x38                           # 1.0
        ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1)
        want = np.zeros((M, N))
        want[m, :] = (float(sa[k // 128, m]) * sb[k // 128, np.arange(N) // 128].astype(np.float64)
                      * db[:, k])
        assert np.array_equal(ref, want)


def test_hand_4x4_product(orc):
    with open(os.path.join(GOLDEN, "hand_4x4.json")) as f:
        g = json.load(f)
    A = np.array(g["A"], dtype=np.float32)
    B = np.array(g["B"], dtype=np.float32)
    qa, sa = orc.quantize(A, 128)
    qb, sb = orc.quantize(B, 128)
    ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=128)
    dot = np.array(g["block_128x128"]["int_dot"], dtype=np.float64)
    assert np.array_equal(ref, dot * float(sa[0, 0]) * float(sb[0, 0]))
    assert np.allclose(ref, np.array(g["block_128x128"]["ref"]), rtol=0, atol=1e-9)
    qa1, sa1 = orc.quantize(A, 1)
    ref1 = orc.gemm_nt(qa1, sa1, qb, sb, a_block_rows=1)
    assert np.allclose(ref1[3], g["a_block_1x128"]["ref_row3"], rtol=0, atol=1e-8)
    assert np.array_equal(ref1[:3], ref[:3])


def test_power_of_two_scale_exchange_is_bit_identical(orc):
    g = np.random.default_rng(5)
    qa, qb = _rand_codes(g, (7, 384)), _rand_codes(g, (9, 384))
    sa, sb = _rand_scales(g, (3, 7)), _rand_scales(g, (3, 1))
    ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1)
    for j in (-7, 4):
        ref2 = orc.gemm_nt(qa, sa * np.float32(2.0 ** j), qb, sb * np.float32(2.0 ** -j),
                           a_block_rows=1)
        assert np.array_equal(ref, ref2)
    # uniform scales factor out of the integer-code product
    s_a, s_b = np.float32(0.125), np.float32(0.0625)
    ref3 = orc.gemm_nt(qa, np.full((3, 7), s_a), qb, np.full((3, 1), s_b), a_block_rows=1)
    dd = exact.torch_decode(qa) @ exact.torch_decode(qb).T
    assert np.array_equal(ref3, dd * float(s_a) * float(s_b))


def test_points_equal_full_product(orc):
    g = np.random.default_rng(6)
    qa, qb = _rand_codes(g, (40, 256)), _rand_codes(g, (300, 256))
    sa, sb = _rand_scales(g, (2, 40)), _rand_scales(g, (2, 3))
    ref = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1)
    pm = g.integers(0, 40, size=100)
    pn = g.integers(0, 300, size=100)
    pts = orc.gemm_nt_points(qa, sa, qb, sb, pm, pn, a_block_rows=1)
    assert np.array_equal(pts, ref[pm, pn])


@pytest.mark.parametrize("br", [1, 128])
def test_grouped_equals_per_expert_matmul(orc, br):
    G, N, K = 3, 136, 256
    r = datagen.moe_routing(num_tokens=40, num_experts=G, topk=2, align=128, seed=8)
    mi = r["m_indices"]
    M = mi.shape[0]
    x = datagen.normal((40, K), 1.0, seed=8, stream=1)
    a = datagen.gather_rows(x, r["row_token"])
    qa, sa = orc.quantize(a, br)
    w = datagen.normal((G * N, K), 0.02, seed=8, stream=2)
    qbs, sbs = [], []
    for e in range(G):
        q, s = orc.quantize(w[e * N:(e + 1) * N], 128)
        qbs.append(q)
        sbs.append(s)
    qb, sb = np.stack(qbs), np.stack(sbs)
    ref = orc.grouped_gemm_contig(qa, sa, qb, sb, mi, a_block_rows=br)
    pad = mi < 0
    assert np.all(ref[pad] == 0.0)
    for e in range(G):
        rows = np.nonzero(mi == e)[0]
        sa_rows = sa[:, rows // br] if br == 1 else None
        da = exact.torch_decode(qa[rows])
        kbi = np.arange(K) // 128
        if br == 1:
            sa_el = sa_rows.astype(np.float64)[kbi][:, :].T
        else:
            sa_el = sa.astype(np.float64)[kbi[None, :], (rows // 128)[:, None]]
        db = exact.torch_decode(qb[e])
        sb_el = sb[e].astype(np.float64)[kbi[None, :], (np.arange(N) // 128)[:, None]]
        want = (da * sa_el) @ (db * sb_el).T
        rms = np.sqrt(np.mean(want ** 2))
        assert np.max(np.abs(ref[rows] - want)) <= 1e-12 * rms
        # a single expert reduces to the dense product
        dense = orc.gemm_nt(qa[rows], np.ascontiguousarray(
            sa[:, rows // br] if br == 1 else sa[:, rows[::128] // 128]), qb[e], sb[e],
            a_block_rows=br)
        assert np.array_equal(dense, ref[rows])


def test_grouped_rejects_bad_expert_id(orc):
    qa = np.zeros((128, 128), np.uint8)
    qb = np.zeros((2, 128, 128), np.uint8)
    mi = np.zeros(128, np.int32)
    mi[5] = 2
    with pytest.raises(ValueError):
        orc.grouped_gemm_contig(qa, np.ones((1, 1), np.float32), qb,
                                np.ones((2, 1, 1), np.float32), mi)
