"""GPU parity of the balanced grouped GEMM (dg_fp8_grouped_gemm_contig_balanced:
the grouped MoE GEMM of the pzsr.cn DeepGEMM page s2.3, s3.2, s3.3 with the
(tile, K block) work shared out over one persistent workgroup per compute
unit, after the persistent thread blocks of the hotelren.com DeepGEMM
walk-through s5.6).  Reference: the FP64 oracle, as for the one-workgroup-
per-tile call; padding rows must be exact zeros.  The shapes are chosen so
that tiles are split between workgroups (pieces summed through the
workspace), and one case has more than two waves of tiles (whole tiles
first, then the shared ones)."""
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


def operands(orc, tokens, G, N, K, br, seed, pad_block=False, drop_expert=None):
    r = datagen.moe_routing(tokens, G, min(2, G), align=128, seed=seed)
    mi, row_token = r["m_indices"], r["row_token"]
    if drop_expert is not None:                  # an expert with no rows at all
        starts = np.concatenate([[0], np.cumsum(r["padded"])])
        keep = np.ones(mi.shape[0], bool)
        keep[starts[drop_expert]:starts[drop_expert + 1]] = False
        mi, row_token = mi[keep], row_token[keep]
    if pad_block:                                # one whole 128-row block of padding
        mi = np.concatenate([mi, np.full(128, -1, np.int32)])
        row_token = np.concatenate([row_token, np.full(128, -1, np.int64)])
    a = datagen.gather_rows(datagen.normal((tokens, K), 1.0, seed=seed, stream=1), row_token)
    qa, sa = orc.quantize(a, br)
    w = datagen.normal((G * N, K), 0.02, seed=seed, stream=2)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, (N + 127) // 128), np.float32)
    for e in range(G):
        qb[e], sb[e] = orc.quantize(w[e * N:(e + 1) * N], 128)
    return qa, sa, qb, sb, mi


def run(dg, qa, sa, qb, sb, mi, br, ws, act="none", residual=None, n_out=None):
    M, N = qa.shape[0], qb.shape[1]
    c = torch.full((M, n_out or N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_grouped_gemm_contig(c, dev(qa), dev(qb), dev(sa), dev(sb), br, dev(mi), act=act,
                                  residual=residual, workspace=ws)
    torch.cuda.synchronize()
    return c


def workspace(dg, M, N, K):
    nb = dg.dg_fp8_grouped_gemm_contig_workspace_bytes(M, N, K)
    assert nb > dg.WORKSPACE_COUNTER_BYTES
    return dg.alloc_workspace(nb)


def counters_zero(dg, ws):
    return int(ws[:dg.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("tokens,G,N,K,pad,drop", [
    (100, 2, 256, 1536, False, None),    # 2 tiles x 12 K blocks on 6 workgroups: 3 pieces each
    (120, 3, 264, 1024, True, 1),        # ragged N, a padding block, an empty expert
    (64, 8, 136, 256, False, None),      # 2 K blocks: whole tiles only, some workgroups idle
    (300, 2, 384, 768, True, None),      # 256- and 128-row tiles, 2 pieces each
])
def test_balanced_small_full_compare(dg, orc, tokens, G, N, K, pad, drop, br):
    qa, sa, qb, sb, mi = operands(orc, tokens, G, N, K, br, seed=tokens + K, pad_block=pad,
                                  drop_expert=drop)
    M = qa.shape[0]
    ws = workspace(dg, M, N, K)
    c = bf16_to_f64(run(dg, qa, sa, qb, sb, mi, br, ws))
    assert counters_zero(dg, ws), "arrival counters must be left zero"
    real = mi >= 0
    assert np.all(c[~real] == 0.0), "padding rows must be zeros"
    ref = orc.grouped_gemm_contig(qa, sa, qb, sb, mi, a_block_rows=br)
    assert_close(c[real], ref[real], rms=float(np.sqrt(np.mean(ref[real] ** 2))),
                 what="balanced %d/%d/%d/%d" % (tokens, G, N, K))


@pytest.mark.parametrize("act,residual", [("swiglu", "in_place"), ("gelu", "separate"),
                                          ("relu", "none"), ("silu", "separate")])
def test_balanced_epilogue(dg, orc, act, residual):
    tokens, G, N, K = 100, 2, 256, 1536
    qa, sa, qb, sb, mi = operands(orc, tokens, G, N, K, 1, seed=31, pad_block=True)
    M = qa.shape[0]
    n_out = N // 2 if act == "swiglu" else N
    c = torch.full((M, n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    res, res_bits = None, None
    if residual != "none":
        r32 = datagen.normal((M, n_out), 0.5, seed=32, stream=0).astype(np.float32)
        res = torch.from_numpy(r32).to(torch.bfloat16).cuda()
        res_bits = res.view(torch.int16).cpu().numpy().view(np.uint16)
        if residual == "in_place":
            c.copy_(res)
            res = c
    ws = workspace(dg, M, N, K)
    dg.dg_fp8_grouped_gemm_contig(c, dev(qa), dev(qb), dev(sa), dev(sb), 1, dev(mi), act=act,
                                  residual=res, workspace=ws)
    torch.cuda.synchronize()
    assert counters_zero(dg, ws)
    got = bf16_to_f64(c)
    real = mi >= 0
    assert np.all(got[~real] == 0.0), "padding rows must be zeros"
    acc = orc.grouped_gemm_contig(qa, sa, qb, sb, mi, a_block_rows=1)
    ref = orc.epilogue(acc[real], act, None if res_bits is None else res_bits[real])
    assert_close(got[real], ref, what="balanced epilogue %s/%s" % (act, residual))


def test_balanced_deterministic_and_workspace_reused(dg, orc):
    """The same inputs give the same bits on every call; one workspace serves
    calls of different shapes in turn (its counters are left zero), and its
    partial tiles need no clearing between calls."""
    ops1 = operands(orc, 300, 4, 512, 1536, 1, seed=41)
    ops2 = operands(orc, 120, 3, 264, 1024, 128, seed=42, pad_block=True)
    M1, M2 = ops1[0].shape[0], ops2[0].shape[0]
    nb = max(dg.dg_fp8_grouped_gemm_contig_workspace_bytes(M1, 512, 1536),
             dg.dg_fp8_grouped_gemm_contig_workspace_bytes(M2, 264, 1024))
    ws = dg.alloc_workspace(nb)
    first = run(dg, *ops1, 1, ws).view(torch.int16).clone()
    second = run(dg, *ops2, 128, ws)
    again = run(dg, *ops1, 1, ws).view(torch.int16)
    assert torch.equal(first, again)
    assert counters_zero(dg, ws)
    ref = orc.grouped_gemm_contig(*ops2, a_block_rows=128)
    real = ops2[4] >= 0
    assert_close(bf16_to_f64(second)[real], ref[real], what="second shape")


def test_balanced_agrees_with_one_tile_per_workgroup(dg, orc):
    """Both calls sum each tile's K blocks in the same order except where the
    balanced call splits it; the sums of the pieces then associate
    differently, so the BF16 outputs agree up to a rounding step."""
    qa, sa, qb, sb, mi = operands(orc, 300, 4, 512, 1536, 1, seed=43)
    M = qa.shape[0]
    ws = workspace(dg, M, 512, 1536)
    cb = bf16_to_f64(run(dg, qa, sa, qb, sb, mi, 1, ws))
    cw = bf16_to_f64(run(dg, qa, sa, qb, sb, mi, 1, None))
    rms = float(np.sqrt(np.mean(cw ** 2)))
    assert np.all(np.abs(cb - cw) <= 2.0 ** -7 * np.abs(cw) + 1e-6 * rms)


def moe_points(mi, N, rng, n_random=2000):
    real_rows = np.nonzero(mi >= 0)[0]
    pm = [rng.choice(real_rows, n_random)]
    pn = [rng.integers(0, N, n_random)]
    tm, tn = tile_points(mi.shape[0], N, 128, 256, rng, rows=real_rows)
    return np.concatenate(pm + [tm]), np.concatenate(pn + [tn])


def sampled_reference(orc, qa, sa, qb, sb, mi, pm, pn, br):
    ref = np.empty(pm.size)
    for e in range(qb.shape[0]):
        sel = mi[pm] == e
        if sel.any():
            ref[sel] = orc.gemm_nt_points(qa, sa, qb[e], sb[e], pm[sel], pn[sel], a_block_rows=br)
    return ref


_WEIGHTS = {}


def moe_weights(orc, G, N, K):
    """Quantised expert weights of the MoE benchmark shapes (kept for the
    other parameters of the test)."""
    if (G, N, K) not in _WEIGHTS:
        w = datagen.normal((G * N, K), 0.02, seed=0, stream=2)
        qb = np.empty((G, N, K), np.uint8)
        sb = np.empty((G, K // 128, N // 128), np.float32)
        for e in range(G):
            qb[e], sb[e] = orc.quantize(w[e * N:(e + 1) * N], 128)
        _WEIGHTS.clear()
        _WEIGHTS[(G, N, K)] = (qb, sb)
    return _WEIGHTS[(G, N, K)]


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("proj,N,K", [("up", 11008, 4096), ("down", 4096, 11008)])
def test_balanced_moe_full_size_sampled(dg, orc, proj, N, K, br):
    """The MoE projections of the benchmark (8 experts, 1024 tokens top-2,
    padded to 128): C starts as NaN, every element must be written and
    finite, padding rows zero; sampled points (one in every 128 x 256 tile
    with real rows) against the oracle."""
    G, tokens = 8, 1024
    r = datagen.moe_routing(tokens, G, 2, align=128, seed=0)
    mi = r["m_indices"]
    M = mi.shape[0]
    if proj == "up":
        a = datagen.gather_rows(datagen.normal((tokens, K), 1.0, seed=0, stream=1), r["row_token"])
    else:
        a = datagen.normal((M, K), 1.0, seed=0, stream=3)
        a[mi < 0] = 0.0
    qa, sa = orc.quantize(a, br)
    qb, sb = moe_weights(orc, G, N, K)
    ws = workspace(dg, M, N, K)
    c = bf16_to_f64(run(dg, qa, sa, qb, sb, mi, br, ws))
    assert counters_zero(dg, ws)
    assert np.all(np.isfinite(c))
    assert np.all(c[mi < 0] == 0.0)
    pm, pn = moe_points(mi, N, np.random.default_rng(1))
    ref = sampled_reference(orc, qa, sa, qb, sb, mi, pm, pn, br)
    assert_close(c[pm, pn], ref, rms=float(np.sqrt(np.mean(ref ** 2))), what="balanced " + proj)


def test_balanced_whole_waves_then_shared(dg, orc):
    """More than two waves of tiles: 4 experts x 2048 rows (32 row tiles of
    256) x 17 column tiles = 544 tiles on at most 256 workgroups, so whole
    tiles go first and the rest is shared out by K block (4 K blocks per
    tile, 4.5 per workgroup: pieces split between neighbours)."""
    G, rows, N, K = 4, 2048, 17 * 256, 512
    mi = np.repeat(np.arange(G, dtype=np.int32), rows)
    M = mi.shape[0]
    qa, sa = orc.quantize(datagen.normal((M, K), 1.0, seed=5, stream=1), 1)
    w = datagen.normal((G * N, K), 0.02, seed=5, stream=2)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, N // 128), np.float32)
    for e in range(G):
        qb[e], sb[e] = orc.quantize(w[e * N:(e + 1) * N], 128)
    ws = workspace(dg, M, N, K)
    c = bf16_to_f64(run(dg, qa, sa, qb, sb, mi, 1, ws))
    assert counters_zero(dg, ws)
    assert np.all(np.isfinite(c))
    rng = np.random.default_rng(2)
    pm, pn = tile_points(M, N, 128, 256, rng)
    pm = np.concatenate([pm, rng.integers(0, M, 1500)])
    pn = np.concatenate([pn, rng.integers(0, N, 1500)])
    ref = sampled_reference(orc, qa, sa, qb, sb, mi, pm, pn, 1)
    assert_close(c[pm, pn], ref, rms=float(np.sqrt(np.mean(ref ** 2))), what="waves")


def test_balanced_calls_on_two_streams_with_distinct_workspaces(dg, orc):
    """Calls are re-entrant: two balanced grouped GEMMs (different shapes)
    launched again and again on two streams of one GPU, each with its own
    workspace, give their single-stream bits on every round."""
    cases = [operands(orc, 100, 2, 256, 1536, 1, seed=51),
             operands(orc, 300, 2, 384, 768, 128, seed=52, pad_block=True)]
    brs = [1, 128]
    wss, eager = [], []
    for (qa, sa, qb, sb, mi), br in zip(cases, brs):
        wss.append(workspace(dg, qa.shape[0], qb.shape[1], qa.shape[1]))
        eager.append(run(dg, qa, sa, qb, sb, mi, br, wss[-1]).view(torch.int16).clone())
    ref0 = orc.grouped_gemm_contig(*cases[0], a_block_rows=1)
    real0 = cases[0][4] >= 0
    assert_close(bf16_to_f64(eager[0].view(torch.bfloat16))[real0], ref0[real0], what="stream case")
    dev_ops = [tuple(dev(x) for x in ops) for ops in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(4):
        outs = [[torch.full((ops[0].shape[0], ops[2].shape[1]), float("nan"), dtype=torch.bfloat16,
                            device="cuda") for _ in range(3)] for ops in cases]
        torch.cuda.synchronize()
        for j in range(3):                              # interleave the launches
            for i, st in enumerate(streams):
                qa, sa, qb, sb, mi = dev_ops[i]
                with torch.cuda.stream(st):
                    dg.dg_fp8_grouped_gemm_contig(outs[i][j], qa, qb, sa, sb, brs[i], mi,
                                                  workspace=wss[i])
        torch.cuda.synchronize()
        for i in range(2):
            for o in outs[i]:
                assert torch.equal(o.view(torch.int16), eager[i]), rnd
            assert counters_zero(dg, wss[i])


def random_layout(rng, G, max_blocks_per_expert=5):
    """m_indices for a random contiguous grouped layout: experts in
    ascending id, each with 0..max_blocks_per_expert 128-row blocks (the
    last one partly padding), and whole padding blocks here and there."""
    ids = []
    for e in range(G):
        if rng.random() < 0.3:
            ids += [-1] * 128                      # a whole padding block
        nb = int(rng.integers(0, max_blocks_per_expert + 1))
        if nb == 0:
            continue                               # an expert with no rows
        real = (nb - 1) * 128 + int(rng.integers(1, 129))
        ids += [e] * real + [-1] * (nb * 128 - real)
    if not ids:
        ids = [0] * 128
    return np.array(ids, dtype=np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts_both_grouped_calls(dg, orc, seed):
    """Random block layouts (runs of 1-5 blocks: pairs and odd 128-row
    tiles; whole padding blocks; empty experts; up to 9 experts) through the
    one-workgroup-per-tile call and the balanced call, both against the
    oracle in full; padding rows must be zeros."""
    rng = np.random.default_rng(700 + seed)
    G = int(rng.integers(2, 10))
    N = int(rng.choice([136, 256, 392, 512]))
    K = int(rng.choice([256, 640, 1024]))
    mi = random_layout(rng, G)
    M = mi.shape[0]
    a = datagen.normal((M, K), 1.0, seed=700 + seed, stream=1)
    a[mi < 0] = 0.0
    br = int(rng.choice([1, 128]))
    qa, sa = orc.quantize(a, br)
    w = datagen.normal((G * N, K), 0.02, seed=700 + seed, stream=2)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, (N + 127) // 128), np.float32)
    for e in range(G):
        qb[e], sb[e] = orc.quantize(w[e * N:(e + 1) * N], 128)
    ref = orc.grouped_gemm_contig(qa, sa, qb, sb, mi, a_block_rows=br)
    real = mi >= 0
    rms = float(np.sqrt(np.mean(ref[real] ** 2)))
    nb = dg.dg_fp8_grouped_gemm_contig_workspace_bytes(M, N, K)
    for ws in (None, dg.alloc_workspace(nb)):
        c = bf16_to_f64(run(dg, qa, sa, qb, sb, mi, br, ws))
        what = "layout %d (%s): G %d M %d N %d K %d" % (seed, "balanced" if ws is not None else
                                                        "per tile", G, M, N, K)
        assert np.all(c[~real] == 0.0), what
        assert_close(c[real], ref[real], rms=rms, what=what)
        if ws is not None:
            assert counters_zero(dg, ws)
