"""GPU masked grouped GEMM parity against the FP64 oracle (pzsr.cn DeepGEMM
page s2.3, s3.2: expert weights batched in one grouped call; the decode-time
layout gives every expert a fixed capacity of max_m rows, masked_m[g] of them
valid).  Valid rows must be within the GEMM tolerance; every other row of C
must keep the sentinel it held before the call, bit for bit."""
import numpy as np
import pytest
import torch

import datagen
from gpu_util import assert_close, bf16_to_f64, dev, need_gpu, tile_points

pytestmark = pytest.mark.gpu

SENTINEL = 0x4B1D  # a BF16 bit pattern no product here produces by accident


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def operands(orc, G, max_m, N, K, br, seed):
    qa = np.empty((G, max_m, K), np.uint8)
    sa = np.empty((G, K // 128, -(-max_m // br)), np.float32)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, -(-N // 128)), np.float32)
    for g in range(G):
        qa[g], sa[g] = orc.quantize(datagen.normal((max_m, K), 1.0, seed=seed, stream=2 * g), br)
        qb[g], sb[g] = orc.quantize(datagen.normal((N, K), 0.02, seed=seed, stream=2 * g + 1), 128)
    return qa, sa, qb, sb


def run(dg, qa, sa, qb, sb, mm, br, workspace):
    G, max_m, _ = qa.shape
    N = qb.shape[1]
    c = torch.full((G, max_m, N), SENTINEL, dtype=torch.int16, device="cuda")
    ws = None
    if workspace:
        n = dg.dg_fp8_grouped_gemm_masked_workspace_bytes(G, max_m, N, qa.shape[2])
        ws = torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda")
    dg.dg_fp8_grouped_gemm_masked(c, dev(qa), dev(qb), dev(sa), dev(sb), br,
                                  dev(np.asarray(mm, np.int32)), workspace=ws)
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16), bf16_to_f64(c)


def check(orc, qa, sa, qb, sb, mm, br, bits, c, what):
    max_m = qa.shape[1]
    clamped = np.clip(np.asarray(mm), 0, max_m).astype(np.int32)
    ref = orc.grouped_gemm_masked(qa, sa, qb, sb, clamped, a_block_rows=br)
    valid = ~np.isnan(ref)
    assert np.all(bits[~valid] == SENTINEL), what + ": rows past masked_m were written"
    if valid.any():
        rms = float(np.sqrt(np.mean(ref[valid] ** 2)))
        assert_close(c[valid], ref[valid], rms=rms, what=what)


CASES = [
    # G, max_m, N, K, br, masks
    (8, 16, 512, 1024, 1, [16, 0, 3, 9, 16, 1, 12, 5]),
    (4, 37, 264, 384, 1, [37, 20, 0, 1]),
    (3, 64, 1024, 512, 128, [64, 33, 17]),
    (2, 100, 256, 256, 1, [100, 70]),        # two 64-row chunks per group
    (8, 1, 4096, 2048, 1, [1, 0, 1, 1, 0, 1, 1, 1]),
    (5, 32, 136, 1280, 128, [-5, 40, 32, 31, 0]),  # out-of-range masks count as clamped
    (2, 200, 512, 512, 128, [200, 150]),     # four chunks, rows past 128: second A scale block
]


@pytest.mark.parametrize("workspace", [False, True])
@pytest.mark.parametrize("G,max_m,N,K,br,mm", CASES)
def test_masked_matches_oracle(dg, orc, G, max_m, N, K, br, mm, workspace):
    qa, sa, qb, sb = operands(orc, G, max_m, N, K, br, seed=G * 31 + max_m)
    bits, c = run(dg, qa, sa, qb, sb, mm, br, workspace)
    check(orc, qa, sa, qb, sb, mm, br, bits, c,
          "masked %s ws=%s" % ((G, max_m, N, K, br), workspace))


def test_masked_split_k_is_deterministic_and_matches_the_plain_call(dg, orc):
    G, max_m, N, K = 8, 16, 1024, 4096
    assert dg.dg_fp8_grouped_gemm_masked_workspace_bytes(G, max_m, N, K) > 0   # plans split-K
    qa, sa, qb, sb = operands(orc, G, max_m, N, K, 1, seed=7)
    mm = [16, 15, 1, 0, 8, 16, 2, 11]
    b1, c1 = run(dg, qa, sa, qb, sb, mm, 1, True)
    b2, _ = run(dg, qa, sa, qb, sb, mm, 1, True)
    assert np.array_equal(b1, b2)
    check(orc, qa, sa, qb, sb, mm, 1, b1, c1, "masked split-K")
    # each group's valid rows equal the dense small-M call on that group
    for g in (0, 4):
        m = mm[g]
        cd = torch.empty((m, N), dtype=torch.bfloat16, device="cuda")
        dg.dg_fp8_gemm_nt(cd, dev(qa[g, :m]), dev(qb[g]), dev(np.ascontiguousarray(sa[g, :, :m])),
                          dev(sb[g]), 1)
        torch.cuda.synchronize()
        ref = orc.gemm_nt(qa[g, :m], np.ascontiguousarray(sa[g, :, :m]), qb[g], sb[g],
                          a_block_rows=1)
        assert_close(bf16_to_f64(cd), ref, what="dense group %d" % g)
        assert_close(c1[g, :m], ref, what="masked group %d" % g)


def test_all_groups_empty_writes_nothing(dg, orc):
    qa, sa, qb, sb = operands(orc, 4, 16, 256, 256, 1, seed=9)
    bits, _ = run(dg, qa, sa, qb, sb, [0, 0, 0, 0], 1, True)
    assert np.all(bits == SENTINEL)


@pytest.mark.parametrize("N,K", [(11008, 4096), (4096, 11008)])
def test_masked_decode_moe_full_size_sampled(dg, orc, N, K):
    """The bench's decode MoE workload: 8 experts with a capacity of 32
    rows, 64 tokens routed top-2 (the routed counts are the masks), up and
    down projections; 2000 sampled valid outputs against the oracle, every
    row past the counts untouched."""
    G, cap = 8, 32
    r = datagen.moe_routing(64, G, 2, align=1, seed=0)
    mm = np.minimum(r["counts"], cap).astype(np.int32)
    qa = np.empty((G, cap, K), np.uint8)
    sa = np.empty((G, K // 128, cap), np.float32)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, N // 128), np.float32)
    w = datagen.normal((G * N, K), 0.02, seed=0, stream=2)
    for g in range(G):
        qa[g], sa[g] = orc.quantize(datagen.normal((cap, K), 1.0, seed=0, stream=10 + g), 1)
        qb[g], sb[g] = orc.quantize(w[g * N:(g + 1) * N], 128)
    bits, c = run(dg, qa, sa, qb, sb, mm, 1, True)
    for g in range(G):
        assert np.all(bits[g, mm[g]:] == SENTINEL)
    rng = np.random.default_rng(3)
    pg = rng.integers(0, G, 2000)
    pm = (rng.random(2000) * mm[pg]).astype(np.int64)
    pn = rng.integers(0, N, 2000)
    for g in range(G):                              # one point per group and 128-column tile
        if mm[g] > 0:
            tm, tn = tile_points(int(mm[g]), N, 64, 128, rng)
            pg = np.concatenate([pg, np.full(tm.size, g)])
            pm = np.concatenate([pm, tm])
            pn = np.concatenate([pn, tn])
    ref = np.empty(pm.size)
    for g in range(G):
        sel = pg == g
        ref[sel] = orc.gemm_nt_points(qa[g], sa[g], qb[g], sb[g], pm[sel], pn[sel], a_block_rows=1)
    assert_close(c[pg, pm, pn], ref, rms=float(np.sqrt(np.mean(ref ** 2))),
                 what="masked decode MoE %dx%d" % (N, K))
