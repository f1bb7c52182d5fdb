"""Pins for the oracle's K-grouped product (pzsr.cn DeepGEMM page s3.2:
grouped GEMM along K, the MoE weight-gradient layout): each group's output is
the plain product restricted to its K range, so (i) one group over all of K
is the plain product, (ii) the groups' outputs sum to the plain product
(linearity over disjoint K ranges), (iii) an empty range gives zeros, and
(iv) each group equals the plain product of the sliced operands and scales."""
import numpy as np
import pytest

import datagen


def operands(orc, M, N, K, seed=0):
    qa, sa = orc.quantize(datagen.normal((M, K), 1.0, seed=seed, stream=0), 1)
    qb, sb = orc.quantize(datagen.normal((N, K), 1.0, seed=seed, stream=1), 128)
    return qa, sa, qb, sb


def test_single_group_is_the_plain_product(orc):
    qa, sa, qb, sb = operands(orc, 9, 136, 512)
    out = orc.grouped_gemm_k(qa, sa, qb, sb, [0, 512])
    assert np.array_equal(out[0], orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1))


def test_groups_sum_to_the_plain_product_and_empty_groups_are_zero(orc):
    M, N, K = 7, 264, 1280
    qa, sa, qb, sb = operands(orc, M, N, K, seed=3)
    ko = [0, 256, 256, 896, 1280]
    out = orc.grouped_gemm_k(qa, sa, qb, sb, ko)
    assert np.all(out[1] == 0.0)
    full = orc.gemm_nt(qa, sa, qb, sb, a_block_rows=1)
    assert np.allclose(out.sum(axis=0), full, rtol=1e-12, atol=1e-12)


def test_each_group_is_the_product_of_its_slices(orc):
    M, N, K = 5, 256, 768
    qa, sa, qb, sb = operands(orc, M, N, K, seed=4)
    ko = [0, 384, 768]
    out = orc.grouped_gemm_k(qa, sa, qb, sb, ko)
    for g in range(2):
        k0, k1 = ko[g], ko[g + 1]
        ref = orc.gemm_nt(np.ascontiguousarray(qa[:, k0:k1]), np.ascontiguousarray(sa[k0 // 128:k1 // 128]),
                          np.ascontiguousarray(qb[:, k0:k1]), np.ascontiguousarray(sb[k0 // 128:k1 // 128]),
                          a_block_rows=1)
        assert np.array_equal(out[g], ref)


def test_rejects_unaligned_ranges(orc):
    qa, sa, qb, sb = operands(orc, 4, 128, 256)
    with pytest.raises(ValueError):
        orc.grouped_gemm_k(qa, sa, qb, sb, [0, 100, 256])
