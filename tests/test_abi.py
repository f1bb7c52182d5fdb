"""The C-ABI library loads, exports every entry point declared in
include/dg.h, and rejects bad arguments on the host before any HIP call
(these calls enqueue nothing and need no GPU)."""
import ctypes
import functools
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "dg.h")


@pytest.fixture(scope="module")
def dg():
    import fp8_block_scaled_dg_amd as m
    return m


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for need in ("dg_quantize_fp8_block", "dg_fp8_gemm_nt", "dg_fp8_grouped_gemm_contig",
                 "dg_abi_version", "dg_status_string", "dg_fp8_gemm_nt_workspace_bytes",
                 "dg_get_mk_alignment_for_contiguous_layout", "dg_fp8_gemm_nt_fused_a",
                 "dg_quantize_fp8_block_ue8m0", "dg_fp8_gemm_nt_ue8m0", "dg_fp8_gemm_nt_epilogue",
                 "dg_transpose_fp8", "dg_fp8_gemm", "dg_fp8_gemm_workspace_bytes",
                 "dg_fp8_grouped_gemm_k", "dg_fp8_grouped_gemm_masked",
                 "dg_fp8_grouped_gemm_masked_workspace_bytes", "dg_fp8_grouped_gemm_contig_ue8m0",
                 "dg_fp8_grouped_gemm_contig_epilogue", "dg_fp8_grouped_gemm_masked_epilogue",
                 "dg_fp8_grouped_gemm_contig_balanced",
                 "dg_fp8_grouped_gemm_contig_workspace_bytes"):
        assert need in names


def test_library_exports_every_declared_symbol(dg):
    lib = ctypes.CDLL(dg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(dg):
    assert dg.lib.dg_abi_version() == 3 == dg.ABI_VERSION
    for st in range(0, 8):
        assert dg.status_string(st) and dg.status_string(st) != "unknown status"
    assert dg.status_string(99) == "unknown status"
    assert dg.get_mk_alignment_for_contiguous_layout() == 128


P = ctypes.c_void_p(0x10000)   # dummy, 16-byte aligned, never dereferenced
P1 = ctypes.c_void_p(0x10001)  # misaligned


def q(lib, qp=P, sp=P, xp=P, rows=128, cols=128, br=128):
    return lib.dg_quantize_fp8_block(qp, sp, xp, rows, cols, br, None)


def test_quantize_validation(dg):
    lib = dg.lib
    assert q(lib, qp=None) == 1
    assert q(lib, sp=None) == 1
    assert q(lib, xp=None) == 1
    assert q(lib, br=64) == 3
    assert q(lib, rows=0) == 2
    assert q(lib, cols=0) == 2
    assert q(lib, cols=24) == 2          # cols % 16
    assert q(lib, rows=-5) == 2
    assert q(lib, rows=128 * 70000) == 2  # grid limit
    assert q(lib, xp=P1) == 4
    assert q(lib, qp=P1) == 4


def g(lib, c=P, a=P, b=P, sa=P, sb=P, br=128, M=256, N=256, K=256, ws=None, wsb=0):
    return lib.dg_fp8_gemm_nt(c, a, b, sa, sb, br, M, N, K, ws, wsb, None)


def test_gemm_validation(dg):
    lib = dg.lib
    for kw in ("c", "a", "b", "sa", "sb"):
        assert g(lib, **{kw: None}) == 1
    assert g(lib, br=2) == 3
    assert g(lib, M=0) == 2
    assert g(lib, N=4) == 2
    assert g(lib, N=260) == 2            # N % 8
    assert g(lib, K=64) == 2
    assert g(lib, K=200) == 2            # K % 128
    assert g(lib, M=70000, K=65536 + 128) == 2   # 32-bit offsets
    assert g(lib, a=P1) == 4
    assert g(lib, sa=ctypes.c_void_p(0x10002)) == 4


def gg(lib, mi=P, G=2, M=256, N=256, K=256, br=1):
    return lib.dg_fp8_grouped_gemm_contig(P, P, P, P, P, br, mi, G, M, N, K, None)


def test_grouped_validation(dg):
    lib = dg.lib
    assert gg(lib, mi=None) == 1
    assert gg(lib, G=0) == 3
    assert gg(lib, M=200) == 2            # M % 128
    assert gg(lib, K=100) == 2
    assert gg(lib, mi=ctypes.c_void_p(0x10002)) == 4


def test_small_m_workspace_too_small_is_rejected(dg):
    lib = dg.lib
    need = dg.dg_fp8_gemm_nt_workspace_bytes(16, 4096, 4096)
    assert need > 16                      # this shape plans a split-K reduction
    assert g(lib, M=16, N=4096, K=4096, ws=P, wsb=16) == 5
    assert g(lib, M=16, N=4096, K=4096, ws=P1, wsb=need) == 4   # misaligned workspace


def test_workspace_query_is_host_only(dg):
    assert dg.dg_fp8_gemm_nt_workspace_bytes(1, 4096, 4096) >= 0
    assert dg.dg_fp8_gemm_nt_workspace_bytes(0, 4096, 4096) == 0


def gf(lib, c=P, a=P, b=P, sb=P, M=16, N=256, K=256, ws=None, wsb=0, bf16=False):
    fn = lib.dg_fp8_gemm_nt_fused_a_bf16 if bf16 else lib.dg_fp8_gemm_nt_fused_a
    return fn(c, a, b, sb, M, N, K, ws, wsb, None)


@pytest.mark.parametrize("bf16", [False, True])
def test_fused_a_validation(dg, bf16):
    lib = dg.lib
    assert dg.FUSED_A_MAX_M == 64
    assert gf(lib, M=64, bf16=bf16, a=P1) == 4     # 64 rows pass the shape checks
    call = functools.partial(gf, bf16=bf16)
    for kw in ("c", "a", "b", "sb"):
        assert call(lib, **{kw: None}) == 1
    assert call(lib, M=0) == 2
    assert call(lib, M=dg.FUSED_A_MAX_M + 1) == 2   # decode batches only
    assert call(lib, N=4) == 2
    assert call(lib, N=260) == 2            # N % 8
    assert call(lib, K=200) == 2            # K % 128
    assert call(lib, N=65536, K=65536 + 128) == 2   # N*K >= 2^32
    assert call(lib, a=P1) == 4
    assert call(lib, sb=ctypes.c_void_p(0x10002)) == 4
    need = dg.dg_fp8_gemm_nt_workspace_bytes(16, 4096, 4096)
    assert call(lib, M=16, N=4096, K=4096, ws=P, wsb=16) == 5
    assert call(lib, M=16, N=4096, K=4096, ws=P1, wsb=need) == 4


def test_ue8m0_validation(dg):
    lib = dg.lib
    assert lib.dg_quantize_fp8_block_ue8m0(None, P, P, 128, 128, 128, None) == 1
    assert lib.dg_quantize_fp8_block_ue8m0(P, P, P, 128, 128, 64, None) == 3
    assert lib.dg_quantize_fp8_block_ue8m0(P, P, P, 128, 24, 128, None) == 2
    assert lib.dg_quantize_fp8_block_ue8m0(P, ctypes.c_void_p(0x10002), P, 128, 128, 128,
                                           None) == 4

    def ge(c=P, a=P, b=P, sfa=P, sfb=P, br=128, M=256, N=256, K=256):
        return lib.dg_fp8_gemm_nt_ue8m0(c, a, b, sfa, sfb, br, M, N, K, None, 0, None)
    for kw in ("c", "a", "b", "sfa", "sfb"):
        assert ge(**{kw: None}) == 1
    assert ge(br=2) == 3
    assert ge(M=0) == 2 and ge(N=260) == 2 and ge(K=200) == 2
    assert ge(a=P1) == 4 and ge(sfb=ctypes.c_void_p(0x10002)) == 4


def test_epilogue_validation(dg):
    lib = dg.lib

    def ge(act=0, res=None, **kw):
        args = dict(c=P, a=P, b=P, sa=P, sb=P, br=128, M=256, N=256, K=256)
        args.update(kw)
        return lib.dg_fp8_gemm_nt_epilogue(args["c"], args["a"], args["b"], args["sa"], args["sb"],
                                           args["br"], args["M"], args["N"], args["K"], act, res,
                                           None, 0, None)
    assert ge(act=5) == 3 and ge(act=-1) == 3
    assert ge(res=P1) == 4
    assert ge(c=None) == 1
    assert ge(N=260) == 2


def test_layouts_transpose_and_k_grouped_validation(dg):
    lib = dg.lib
    assert lib.dg_transpose_fp8(None, P, 16, 16, None) == 1
    assert lib.dg_transpose_fp8(ctypes.c_void_p(0x20000), P, 24, 16, None) == 2
    assert lib.dg_transpose_fp8(ctypes.c_void_p(0x20000), P1, 16, 16, None) == 4
    assert lib.dg_transpose_fp8(P, ctypes.c_void_p(0x10010), 64, 64, None) == 3   # overlap

    def gl(layout=1, ws=None, wsb=0, M=256, N=256, K=256):
        return lib.dg_fp8_gemm(P, P, P, P, P, 128, M, N, K, layout, ws, wsb, None)
    assert gl(layout=4) == 3 and gl(layout=-1) == 3
    need = dg.dg_fp8_gemm_workspace_bytes(256, 256, 256, "tn")
    # the counter region first (never written by the transposes), then the copies
    assert need == dg.WORKSPACE_COUNTER_BYTES + 2 * 256 * 256
    assert gl() == 5                                   # transposed operands need a workspace
    assert gl(ws=P, wsb=16) == 5
    assert gl(ws=P, wsb=2 * 256 * 256) == 5            # copies without the counter region
    assert gl(ws=P1, wsb=need) == 4
    assert gl(M=264, ws=P, wsb=1 << 30) == 2            # A given [K][M] needs M % 16 == 0
    assert dg.dg_fp8_gemm_workspace_bytes(256, 256, 256, "nt") == \
        dg.dg_fp8_gemm_nt_workspace_bytes(256, 256, 256)
    # small M: the split-K region (counters + partials) ahead of the copies
    nt = dg.dg_fp8_gemm_nt_workspace_bytes(16, 4096, 4096)
    assert nt > dg.WORKSPACE_COUNTER_BYTES
    assert dg.dg_fp8_gemm_workspace_bytes(16, 4096, 4096, "nn") == nt + 4096 * 4096
    assert dg.dg_fp8_gemm_workspace_bytes(16, 4096, 4096, "tt") == nt + 16 * 4096

    def gk(ko=P, G=2, M=256, N=256, K=256):
        return lib.dg_fp8_grouped_gemm_k(P, P, P, P, P, 128, ko, G, M, N, K, None)
    assert gk(ko=None) == 1
    assert gk(G=0) == 3
    assert gk(ko=ctypes.c_void_p(0x10004)) == 4
    assert gk(K=200) == 2


def test_masked_grouped_validation(dg):
    lib = dg.lib

    def gm(c=P, mm=P, G=8, max_m=16, N=512, K=512, br=1, ws=None, wsb=0):
        return lib.dg_fp8_grouped_gemm_masked(c, P, P, P, P, br, mm, G, max_m, N, K, ws, wsb,
                                              None)
    assert gm(c=None) == 1 and gm(mm=None) == 1
    assert gm(G=0) == 3 and gm(br=64) == 3
    assert gm(max_m=0) == 2 and gm(N=100) == 2 and gm(K=200) == 2
    assert gm(mm=ctypes.c_void_p(0x10002)) == 4 and gm(c=P1) == 4
    need = dg.dg_fp8_grouped_gemm_masked_workspace_bytes(8, 16, 512, 4096)
    assert need > 16                      # this shape plans a split-K reduction
    assert need == dg.dg_fp8_grouped_gemm_masked_workspace_bytes(8, 16, 512, 4096)
    assert gm(K=4096, ws=P, wsb=16) == 5
    assert gm(K=4096, ws=P1, wsb=need) == 4
    assert dg.dg_fp8_grouped_gemm_masked_workspace_bytes(0, 16, 512, 4096) == 0


def test_grouped_epilogue_validation(dg):
    lib = dg.lib
    MI = ctypes.c_void_p(0x10000)

    def ge(act=0, res=None, M=256):
        return lib.dg_fp8_grouped_gemm_contig_epilogue(P, P, P, P, P, 1, MI, 4, M, 512, 512, act,
                                                       res, None)
    assert ge(act=5) == 3 and ge(act=-1) == 3
    assert ge(res=P1) == 4
    assert ge(M=200) == 2

    def me(act=0, res=None):
        return lib.dg_fp8_grouped_gemm_masked_epilogue(P, P, P, P, P, 1, MI, 8, 16, 512, 512, act,
                                                       res, None, 0, None)
    assert me(act=7) == 3 and me(res=P1) == 4


def test_grouped_balanced_validation(dg):
    """The balanced grouped GEMM validates like the epilogue call, then its
    workspace: a too-small one is rejected, a misaligned one too, and none
    at all means the one-workgroup-per-tile call."""
    lib = dg.lib
    MI = ctypes.c_void_p(0x10000)

    def gb(mi=MI, G=8, M=2432, N=4096, K=11008, act=0, res=None, ws=None, wsb=0):
        return lib.dg_fp8_grouped_gemm_contig_balanced(P, P, P, P, P, 1, mi, G, M, N, K, act, res,
                                                       ws, wsb, None)
    assert gb(mi=None) == 1 and gb(G=0) == 3 and gb(act=5) == 3
    assert gb(M=200) == 2 and gb(K=100) == 2 and gb(res=P1) == 4
    assert gb(mi=ctypes.c_void_p(0x10002)) == 4
    need = dg.dg_fp8_grouped_gemm_contig_workspace_bytes(2432, 4096, 11008)
    # counters, then two partial 256 x 256 FP32 tiles for each of at most 256 workers
    assert need == dg.WORKSPACE_COUNTER_BYTES + 2 * 256 * 256 * 256 * 4
    assert gb(ws=P, wsb=need - 1) == 5
    assert gb(ws=P1, wsb=need) == 4
    # small problems need fewer slots: 2 row blocks x 1 column tile x 8 K blocks
    small = dg.dg_fp8_grouped_gemm_contig_workspace_bytes(256, 256, 1024)
    assert small == dg.WORKSPACE_COUNTER_BYTES + 2 * 4 * 256 * 256 * 4
    # shapes it does not share out, and invalid ones: no workspace
    assert dg.dg_fp8_grouped_gemm_contig_workspace_bytes(513 * 128, 256, 1024) == 0
    assert dg.dg_fp8_grouped_gemm_contig_workspace_bytes(128, 2049 * 256, 1024) == 0
    assert dg.dg_fp8_grouped_gemm_contig_workspace_bytes(256, 256, 8193 * 128) == 0
    assert dg.dg_fp8_grouped_gemm_contig_workspace_bytes(200, 256, 1024) == 0
    assert dg.dg_fp8_grouped_gemm_contig_workspace_bytes(256, 256, 100) == 0


def test_grouped_ue8m0_validation(dg):
    lib = dg.lib
    MI = ctypes.c_void_p(0x10000)

    def gu(mi=MI, G=4, M=256, K=512, br=1):
        return lib.dg_fp8_grouped_gemm_contig_ue8m0(P, P, P, P, P, br, mi, G, M, 512, K, None)
    assert gu(mi=None) == 1 and gu(G=0) == 3 and gu(br=7) == 3
    assert gu(M=200) == 2 and gu(K=100) == 2
    assert gu(mi=ctypes.c_void_p(0x10002)) == 4


def test_noalloc_validation(dg):
    """The no-allocation GEMM validates like dg_fp8_gemm_nt before any HIP
    call."""
    lib = dg.lib

    def gn(c=P, a=P, b=P, sa=P, sb=P, br=1, M=64, N=4096, K=4096):
        return lib.dg_fp8_gemm_nt_noalloc(c, a, b, sa, sb, br, M, N, K, None)
    for kw in ("c", "a", "b", "sa", "sb"):
        assert gn(**{kw: None}) == 1
    assert gn(br=2) == 3
    assert gn(M=0) == 2 and gn(N=260) == 2 and gn(K=200) == 2
    assert gn(a=P1) == 4
    # every small-M plan fits the static scratch
    for M in (1, 5, 16, 17, 33, 64):
        for N in (8, 1000, 4096, 7168, 8192, 16384, 24576, 65536):
            assert dg.dg_fp8_gemm_nt_workspace_bytes(M, N, 16384) <= dg.NOALLOC_SCRATCH_BYTES
