"""Every entry point captured into a HIP graph: replayed several times, with
eager launches and synchronisations between the replays and the outputs
zeroed before each, a graph must reproduce the eager result bit for bit.
The calls enqueue kernels only (no memsets), and the split-K counters are
left zeroed by every call, which this exercises across replays."""
import numpy as np
import pytest
import torch

import datagen
from gpu_util import dev, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def check_graph(make_outputs, run):
    """run(outs) enqueues the operation writing into the tensors outs."""
    eager = make_outputs()
    run(eager)
    torch.cuda.synchronize()
    eager = [t.clone() for t in eager]
    sets = [make_outputs() for _ in range(2)]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for outs in sets:
                run(outs)
    torch.cuda.synchronize()
    for rep in range(3):
        for outs in sets:
            for t in outs:
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for outs in sets:
            for t, e in zip(outs, eager):
                assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), "replay %d" % rep
        again = make_outputs()                      # eager work between replays
        run(again)
        torch.cuda.synchronize()
        for t, e in zip(again, eager):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8))


def bf16(M, N):
    return lambda: [torch.empty((M, N), dtype=torch.bfloat16, device="cuda")]


def quantised(orc, M, N, K, br=1, seed=0):
    qa, sa = orc.quantize(datagen.normal((M, K), 1.0, seed=seed, stream=0), br)
    qb, sb = orc.quantize(datagen.normal((N, K), 0.02, seed=seed, stream=1), 128)
    return dev(qa), dev(sa), dev(qb), dev(sb)


@pytest.mark.parametrize("br", [128, 1])
def test_graph_quantisers(dg, br):
    x = dev(datagen.normal((300, 1152), 1.0, seed=2))
    nkb, nrb = 9, -(-300 // br)

    def outs():
        return [torch.empty((300, 1152), dtype=torch.uint8, device="cuda"),
                torch.empty((nkb, nrb), dtype=torch.float32, device="cuda"),
                torch.empty((300, 1152), dtype=torch.uint8, device="cuda"),
                torch.empty((3, nrb), dtype=torch.int32, device="cuda")]

    def run(o):
        dg.dg_quantize_fp8_block(o[0], o[1], x, br)
        dg.dg_quantize_fp8_block_ue8m0(o[2], o[3], x, br)
    check_graph(outs, run)


@pytest.mark.parametrize("M,N,K", [(16, 4096, 4096), (1, 24576, 1536), (8, 1032, 1024)])
def test_graph_fused_activation_quantisation(dg, orc, M, N, K):
    a = dev(datagen.normal((M, K), 1.0, seed=3, stream=0))
    _, _, qb, sb = quantised(orc, 1, N, K)
    wsb = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")
    check_graph(bf16(M, N), lambda o: dg.dg_fp8_gemm_nt_fused_a(o[0], a, qb, sb, workspace=ws))


@pytest.mark.parametrize("M,N,K,act", [(300, 520, 640, "swiglu"), (12, 2056, 16384, "silu"),
                                       (4, 1032, 1024, "gelu")])
def test_graph_epilogue_with_residual(dg, orc, M, N, K, act):
    qa, sa, qb, sb = quantised(orc, M, N, K, seed=4)
    n_out = N // 2 if act == "swiglu" else N
    r = dev(datagen.normal((M, n_out), 1.0, seed=5)).to(torch.bfloat16)
    wsb = dg.dg_fp8_gemm_nt_workspace_bytes(M, N, K)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")
    check_graph(bf16(M, n_out), lambda o: dg.dg_fp8_gemm_nt_epilogue(
        o[0], qa, qb, sa, sb, 1, act=act, residual=r, workspace=ws))


def test_graph_ue8m0_gemm(dg, orc):
    M, N, K = 512, 768, 1024
    qa, ea = orc.quantize_ue8m0(datagen.normal((M, K), 1.0, seed=6, stream=0), 1)
    qb, eb = orc.quantize_ue8m0(datagen.normal((N, K), 0.02, seed=6, stream=1), 128)
    a, b = dev(qa), dev(qb)
    sfa, sfb = dev(orc.pack_ue8m0(ea)), dev(orc.pack_ue8m0(eb))
    check_graph(bf16(M, N), lambda o: dg.dg_fp8_gemm_nt_ue8m0(o[0], a, b, sfa, sfb, 1))


@pytest.mark.parametrize("layout", ["tn", "nn", "tt"])
def test_graph_layouts(dg, orc, layout):
    M, N, K = 256, 384, 512
    qa, sa = orc.quantize(datagen.normal((M, K), 1.0, seed=7, stream=0), 1)
    qb, sb = orc.quantize(datagen.normal((N, K), 0.02, seed=7, stream=1), 128)
    a = dev(np.ascontiguousarray(qa.T) if layout in ("tn", "tt") else qa)
    b = dev(np.ascontiguousarray(qb.T) if layout in ("tn", "nn") else qb)
    sa_d, sb_d = dev(sa), dev(sb)
    ws = torch.zeros(dg.dg_fp8_gemm_workspace_bytes(M, N, K, layout), dtype=torch.uint8,
                     device="cuda")
    check_graph(bf16(M, N), lambda o: dg.dg_fp8_gemm(o[0], a, b, sa_d, sb_d, 1, layout=layout,
                                                     workspace=ws))


def test_graph_k_grouped(dg, orc):
    M, N, K = 300, 520, 1664
    qa, sa, qb, sb = quantised(orc, M, N, K, seed=8)
    ko = torch.tensor([0, 384, 384, 1024, 1664], dtype=torch.int64, device="cuda")
    check_graph(lambda: [torch.empty((4, M, N), dtype=torch.bfloat16, device="cuda")],
                lambda o: dg.dg_fp8_grouped_gemm_k(o[0], qa, qb, sa, sb, 1, ko))


def test_graph_masked_grouped(dg, orc):
    G, max_m, N, K = 8, 16, 1024, 4096
    qa = np.empty((G, max_m, K), np.uint8)
    sa = np.empty((G, K // 128, max_m), np.float32)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, N // 128), np.float32)
    for g in range(G):
        qa[g], sa[g] = orc.quantize(datagen.normal((max_m, K), 1.0, seed=g, stream=0), 1)
        qb[g], sb[g] = orc.quantize(datagen.normal((N, K), 0.02, seed=g, stream=1), 128)
    mm = dev(np.array([16, 0, 5, 16, 9, 1, 12, 3], np.int32))
    n = dg.dg_fp8_grouped_gemm_masked_workspace_bytes(G, max_m, N, K)
    assert n > 0                                  # the split-K plan (counters across replays)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    A, B, SA, SB = dev(qa), dev(qb), dev(sa), dev(sb)
    check_graph(lambda: [torch.zeros((G, max_m, N), dtype=torch.bfloat16, device="cuda")],
                lambda o: dg.dg_fp8_grouped_gemm_masked(o[0], A, B, SA, SB, 1, mm, workspace=ws))


def test_graph_grouped_epilogue_and_ue8m0(dg, orc):
    G, N, K = 4, 512, 640
    r = datagen.moe_routing(200, G, 2, align=128, seed=3)
    mi = r["m_indices"]
    a = datagen.gather_rows(datagen.normal((200, K), 1.0, seed=3, stream=1), r["row_token"])
    M = mi.shape[0]
    qa, sa = orc.quantize(a, 1)
    qa8, ea = orc.quantize_ue8m0(a, 1)
    w = datagen.normal((G * N, K), 0.02, seed=3, stream=2)
    qb = np.empty((G, N, K), np.uint8)
    sb = np.empty((G, K // 128, N // 128), np.float32)
    qb8 = np.empty((G, N, K), np.uint8)
    sfb = []
    for e in range(G):
        qb[e], sb[e] = orc.quantize(w[e * N:(e + 1) * N], 128)
        qb8[e], eb = orc.quantize_ue8m0(w[e * N:(e + 1) * N], 128)
        sfb.append(orc.pack_ue8m0(eb))
    A, B, SA, SB, MI = dev(qa), dev(qb), dev(sa), dev(sb), dev(mi)
    res = torch.randn((M, N // 2), device="cuda").to(torch.bfloat16)
    check_graph(bf16(M, N // 2),
                lambda o: dg.dg_fp8_grouped_gemm_contig(o[0], A, B, SA, SB, 1, MI, act="swiglu",
                                                        residual=res))
    # the balanced call: pieces of split tiles pass through the workspace,
    # whose arrival counters every call leaves zero
    ws = dg.alloc_workspace(dg.dg_fp8_grouped_gemm_contig_workspace_bytes(M, N, K))
    check_graph(bf16(M, N // 2),
                lambda o: dg.dg_fp8_grouped_gemm_contig(o[0], A, B, SA, SB, 1, MI, act="swiglu",
                                                        residual=res, workspace=ws))
    assert int(ws[:dg.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
    A8, B8 = dev(qa8), dev(qb8)
    SFA, SFB = dev(orc.pack_ue8m0(ea)), dev(np.stack(sfb))
    check_graph(bf16(M, N),
                lambda o: dg.dg_fp8_grouped_gemm_contig_ue8m0(o[0], A8, B8, SFA, SFB, 1, MI))
