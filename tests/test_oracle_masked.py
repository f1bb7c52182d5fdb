"""Pins for the oracle's masked grouped product (pzsr.cn DeepGEMM page s2.3
and s3.2: expert weights batched in one grouped call; decode-time layout with
a fixed capacity of max_m rows per expert, masked_m[g] of them valid):
(i) the hand-checked 4x4 product (tests/golden/hand_4x4.json) placed in two
groups with different masks, (ii) a full mask is the plain product of the
group's slices, (iii) a partial mask keeps exactly the first masked_m rows of
it and writes nothing else, (iv) reordering the groups reorders the outputs,
(v) masks outside [0, max_m] are rejected."""
import json
import os

import numpy as np
import pytest

import datagen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def hexcodes(lst, shape):
    return np.array([int(h, 16) for h in lst], dtype=np.uint8).reshape(shape)


def hexf32(lst):
    return np.array([int(h, 16) for h in lst], dtype=np.uint32).view(np.float32)


def operands(orc, G, max_m, N, K, br, seed=0):
    qa = np.empty((G, max_m, K), np.uint8)
    sa = np.empty((G, K // 128, -(-max_m // br)), np.float32)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, -(-N // 128)), np.float32)
    for g in range(G):
        qa[g], sa[g] = orc.quantize(datagen.normal((max_m, K), 1.0, seed=seed, stream=2 * g), br)
        qb[g], sb[g] = orc.quantize(datagen.normal((N, K), 0.02, seed=seed, stream=2 * g + 1), 128)
    return qa, sa, qb, sb


def test_hand_4x4_in_two_masked_groups(orc):
    with open(os.path.join(GOLDEN, "hand_4x4.json")) as f:
        g = json.load(f)["block_128x128"]
    qa = hexcodes(g["qA_hex"], (4, 4))
    qb = hexcodes(g["qB_hex"], (4, 4))
    sa = hexf32(g["sA_hex"]).reshape(1, 1)
    sb = hexf32(g["sB_hex"]).reshape(1, 1)
    want = np.array(g["ref"])
    # group 1 holds A's rows in reverse order and only its first 2 are valid
    QA = np.stack([qa, qa[::-1].copy()])
    out = orc.grouped_gemm_masked(QA, np.stack([sa, sa]), np.stack([qb, qb]),
                                  np.stack([sb, sb]), [4, 2], a_block_rows=128)
    assert np.allclose(out[0], want, rtol=0, atol=1e-9)
    assert np.allclose(out[1, :2], want[[3, 2]], rtol=0, atol=1e-9)
    assert np.all(np.isnan(out[1, 2:]))


@pytest.mark.parametrize("br", [1, 128])
def test_full_mask_is_the_plain_product_of_each_group(orc, br):
    G, max_m, N, K = 3, 5, 136, 384
    qa, sa, qb, sb = operands(orc, G, max_m, N, K, br, seed=1)
    out = orc.grouped_gemm_masked(qa, sa, qb, sb, [max_m] * G, a_block_rows=br)
    for g in range(G):
        assert np.array_equal(out[g], orc.gemm_nt(qa[g], sa[g], qb[g], sb[g], a_block_rows=br))


def test_partial_masks_keep_the_first_rows_only(orc):
    G, max_m, N, K = 4, 7, 128, 256
    qa, sa, qb, sb = operands(orc, G, max_m, N, K, 1, seed=2)
    mm = [0, 3, 7, 1]
    out = orc.grouped_gemm_masked(qa, sa, qb, sb, mm)
    for g in range(G):
        full = orc.gemm_nt(qa[g], sa[g], qb[g], sb[g], a_block_rows=1)
        assert np.array_equal(out[g, :mm[g]], full[:mm[g]])
        assert np.all(np.isnan(out[g, mm[g]:]))


def test_reordering_groups_reorders_outputs(orc):
    G, max_m, N, K = 3, 4, 256, 256
    qa, sa, qb, sb = operands(orc, G, max_m, N, K, 1, seed=3)
    mm = np.array([4, 2, 3], np.int32)
    out = orc.grouped_gemm_masked(qa, sa, qb, sb, mm)
    perm = [2, 0, 1]
    out2 = orc.grouped_gemm_masked(qa[perm], sa[perm], qb[perm], sb[perm], mm[perm])
    assert np.array_equal(np.nan_to_num(out2, nan=7.0), np.nan_to_num(out[perm], nan=7.0))


def test_rejects_masks_outside_the_capacity(orc):
    qa, sa, qb, sb = operands(orc, 2, 4, 128, 128, 1)
    for mm in ([5, 0], [0, -1]):
        with pytest.raises(ValueError):
            orc.grouped_gemm_masked(qa, sa, qb, sb, mm)
