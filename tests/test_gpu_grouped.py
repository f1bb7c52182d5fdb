"""GPU grouped (M-contiguous, MoE) GEMM parity against the FP64 oracle
(pzsr.cn DeepGEMM page s2.3, s3.2, s3.3: experts' rows concatenated along M,
each group padded to the alignment; padding rows carry expert id -1 and must
come out as zeros)."""
import numpy as np
import pytest
import torch

import datagen
from gpu_util import assert_close, bf16_to_f64, dev, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def build(orc, tokens, G, N, K, br, seed, drop_expert=None):
    r = datagen.moe_routing(tokens, G, min(2, G), align=128, seed=seed)
    mi = r["m_indices"].copy()
    if drop_expert is not None:                  # an expert with no rows at all
        starts = np.concatenate([[0], np.cumsum(r["padded"])])
        keep = np.ones(mi.shape[0], bool)
        keep[starts[drop_expert]:starts[drop_expert + 1]] = False
        mi = mi[keep]
        row_token = r["row_token"][keep]
    else:
        row_token = r["row_token"]
    x = datagen.normal((tokens, K), 1.0, seed=seed, stream=1)
    a = datagen.gather_rows(x, row_token)
    qa, sa = orc.quantize(a, br)
    w = datagen.normal((G * N, K), 0.02, seed=seed, stream=2)
    qbs, sbs = [], []
    for e in range(G):
        q, s = orc.quantize(w[e * N:(e + 1) * N], 128)
        qbs.append(q)
        sbs.append(s)
    return qa, sa, np.stack(qbs), np.stack(sbs), mi


def run(dg, qa, sa, qb, sb, mi, br):
    M = qa.shape[0]
    N = qb.shape[1]
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_grouped_gemm_contig(c, dev(qa), dev(qb), dev(sa), dev(sb), br, dev(mi))
    torch.cuda.synchronize()
    return bf16_to_f64(c)


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("tokens,G,N,K", [(40, 3, 264, 256), (300, 4, 512, 384), (64, 8, 136, 128)])
def test_grouped_small_full_compare(dg, orc, tokens, G, N, K, br):
    qa, sa, qb, sb, mi = build(orc, tokens, G, N, K, br, seed=tokens + G)
    ref = orc.grouped_gemm_contig(qa, sa, qb, sb, mi, a_block_rows=br)
    c = run(dg, qa, sa, qb, sb, mi, br)
    real = mi >= 0
    assert np.all(c[~real] == 0.0)
    rms = float(np.sqrt(np.mean(ref[real] ** 2)))
    assert_close(c[real], ref[real], rms=rms, what="grouped %d/%d/%d/%d" % (tokens, G, N, K))


def test_grouped_empty_expert_and_padding_block(dg, orc):
    qa, sa, qb, sb, mi = build(orc, 100, 4, 256, 256, 1, seed=11, drop_expert=2)
    # append one whole 128-row block of padding
    M = qa.shape[0]
    qa = np.concatenate([qa, np.full((128, 256), 0x38, np.uint8)])
    sa_pad = np.ones((sa.shape[0], 128), np.float32)
    sa = np.ascontiguousarray(np.concatenate([sa, sa_pad], axis=1))
    mi = np.concatenate([mi, np.full(128, -1, np.int32)])
    ref = orc.grouped_gemm_contig(qa, sa, qb, sb, mi, a_block_rows=1)
    c = run(dg, qa, sa, qb, sb, mi, 1)
    assert not np.any(mi == 2)
    assert np.all(c[M:] == 0.0) and np.all(c[mi < 0] == 0.0)
    real = mi >= 0
    assert_close(c[real], ref[real], rms=float(np.sqrt(np.mean(ref[real] ** 2))), what="empty")


def test_grouped_single_expert_equals_dense(dg, orc):
    qa, sa, qb, sb, mi = build(orc, 256, 1, 512, 512, 128, seed=12)
    c = run(dg, qa, sa, qb, sb, mi, 128)
    cd = torch.empty((qa.shape[0], 512), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_gemm_nt(cd, dev(qa), dev(qb[0]), dev(sa), dev(sb[0]), 128)
    torch.cuda.synchronize()
    assert np.array_equal(c[mi >= 0], bf16_to_f64(cd)[mi >= 0])


@pytest.mark.parametrize("br", [1, 128])
@pytest.mark.parametrize("proj,N,K", [("up", 11008, 4096), ("down", 4096, 11008)])
def test_grouped_moe_full_size_sampled(dg, orc, proj, N, K, br):
    """8 experts, 1024 tokens routed top-2, rows padded to 128 per expert;
    activations with 1x128 scales (tokens quantised per row before routing)
    and with 128x128 scales (valid too: no block spans two experts).  C
    starts as NaN; every element must be written; sampled points include one
    in every 128-row x 256-column tile that holds real rows."""
    G, tokens = 8, 1024
    r = datagen.moe_routing(tokens, G, 2, align=128, seed=0)
    mi = r["m_indices"]
    M = mi.shape[0]
    if proj == "up":
        x = datagen.normal((tokens, K), 1.0, seed=0, stream=1)
        a = datagen.gather_rows(x, r["row_token"])
    else:
        a = datagen.normal((M, K), 1.0, seed=0, stream=3)
        a[mi < 0] = 0.0
    qa, sa = orc.quantize(a, br)
    w = datagen.normal((G * N, K), 0.02, seed=0, stream=2)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, N // 128), np.float32)
    for e in range(G):
        qb[e], sb[e] = orc.quantize(w[e * N:(e + 1) * N], 128)
    c = run(dg, qa, sa, qb, sb, mi, br)
    assert np.all(np.isfinite(c))
    assert np.all(c[mi < 0] == 0.0)
    g = np.random.default_rng(1)
    real_rows = np.nonzero(mi >= 0)[0]
    pm = [g.choice(real_rows, 2000)]
    pn = [g.integers(0, N, 2000)]
    for blk in range(M // 128):                      # one point per tile with real rows
        rr = real_rows[(real_rows >= blk * 128) & (real_rows < blk * 128 + 128)]
        if rr.size:
            n0 = np.arange(0, N, 256)
            pm.append(g.choice(rr, n0.size))
            pn.append(n0 + g.integers(0, 256, n0.size) % np.minimum(256, N - n0))
    pm, pn = np.concatenate(pm), np.concatenate(pn)
    ref = np.empty(pm.size)
    for e in range(G):
        sel = mi[pm] == e
        if sel.any():
            # rows of one expert: the dense oracle on that expert's weights
            ref[sel] = orc.gemm_nt_points(qa, sa, qb[e], sb[e], pm[sel], pn[sel], a_block_rows=br)
    assert_close(c[pm, pn], ref, rms=float(np.sqrt(np.mean(ref ** 2))), what="moe " + proj)


def test_grouped_at_32bit_offset_limit(dg, orc):
    """Two experts whose N*K is just below 2^32 bytes each (the per-expert
    base is 64-bit, offsets inside an expert 32-bit); rows: expert 0 with 200
    routed rows (2 blocks, the second padded), expert 1 with 128 (1 block)."""
    G, N, K = 2, 32760, 131072
    mi = np.full(384, -1, np.int32)
    mi[:200] = 0
    mi[256:384] = 1
    M = mi.shape[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    qa = torch.randint(0, 0x7E, (M, K), dtype=torch.uint8, device="cuda", generator=g)
    qb = torch.randint(0, 0x7E, (G, N, K), dtype=torch.uint8, device="cuda", generator=g)
    sa = (torch.rand((K // 128, M), device="cuda", generator=g) + 0.5) * 1e-3
    sb = (torch.rand((G, K // 128, N // 128 + 1), device="cuda", generator=g) + 0.5) * 1e-3
    c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    dg.dg_fp8_grouped_gemm_contig(c, qa, qb, sa, sb, 1, dev(mi))
    torch.cuda.synchronize()
    assert torch.all(c[torch.from_numpy(np.nonzero(mi < 0)[0]).cuda()] == 0)
    blocks = [0, (N - 1) // 128]
    cols = np.concatenate([np.arange(b * 128, min(N, b * 128 + 128)) for b in blocks])
    pos = np.concatenate([np.arange(min(N, b * 128 + 128) - b * 128) + i * 128
                          for i, b in enumerate(blocks)])
    for e, rows in ((0, np.array([0, 130, 199])), (1, np.array([256, 300, 383]))):
        qa_h = qa[torch.from_numpy(rows).cuda()].cpu().numpy()
        sa_h = np.ascontiguousarray(sa[:, torch.from_numpy(rows).cuda()].cpu().numpy())
        qb_al = np.zeros((len(blocks) * 128, K), np.uint8)
        qb_al[pos] = qb[e][torch.from_numpy(cols).cuda()].cpu().numpy()
        sb_h = np.ascontiguousarray(sb[e][:, torch.tensor(blocks, device="cuda")].cpu().numpy())
        pm = np.repeat(np.arange(rows.size), cols.size)
        pn = np.tile(np.arange(cols.size), rows.size)
        ref = orc.gemm_nt_points(qa_h, sa_h, qb_al, sb_h, pm, pos[pn], a_block_rows=1)
        got = c[torch.from_numpy(rows[pm]).cuda(), torch.from_numpy(cols[pn]).cuda()]
        assert_close(got.float().cpu().numpy().astype(np.float64), ref,
                     rms=float(np.sqrt(np.mean(ref ** 2))), what="grouped limit e%d" % e)
    del qa, qb, c
    torch.cuda.empty_cache()
