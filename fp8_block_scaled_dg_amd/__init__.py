"""MI355X (gfx950) FP8 E4M3 block-scaled GEMM: Python binding of libdg.so.

Argument marshalling only: every step runs in the HIP kernels of libdg.so
(declared in include/dg.h).  PyTorch provides device memory and the current
stream.  There is no fallback: if the library is missing or fails to load,
importing this package raises.

Entry points (same names as the C ABI):
    dg_quantize_fp8_block(q, scales, x, block_rows)
    dg_fp8_gemm_nt(c, a, b, sa, sb, a_block_rows, workspace=None)
    dg_fp8_grouped_gemm_contig(c, a, b, sa, sb, a_block_rows, m_indices, workspace=None)
    dg_fp8_grouped_gemm_masked(c, a, b, sa, sb, a_block_rows, masked_m, workspace=None)
    (and the UE8M0, fused-A, epilogue, layout and K-grouped entry points)
Conveniences mirroring the DeepGEMM page's Python API (pzsr.cn, s4.1):
    to_fp8(x, block_rows=128) -> (q, scales)
    fp8_gemm_nt(c, a, b, sa, sb, a_block_rows=128)
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libdg.so")

DG_OK = 0
ABI_VERSION = 3
# arrival-counter region at the start of every split-K workspace (dg.h)
WORKSPACE_COUNTER_BYTES = 32768


class DGError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libdg.so not built (%s); run `python fp8_block_scaled_dg_amd/build.py`"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.dg_abi_version.restype = i32
    lib.dg_abi_version.argtypes = []
    lib.dg_status_string.restype = ctypes.c_char_p
    lib.dg_status_string.argtypes = [i32]
    lib.dg_get_mk_alignment_for_contiguous_layout.restype = i32
    lib.dg_get_mk_alignment_for_contiguous_layout.argtypes = []
    lib.dg_quantize_fp8_block.restype = i32
    lib.dg_quantize_fp8_block.argtypes = [vp, vp, vp, i64, i64, i32, vp]
    lib.dg_fp8_gemm_nt_workspace_bytes.restype = ctypes.c_size_t
    lib.dg_fp8_gemm_nt_workspace_bytes.argtypes = [i64, i64, i64]
    lib.dg_fp8_gemm_nt.restype = i32
    lib.dg_fp8_gemm_nt.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, ctypes.c_size_t, vp]
    lib.dg_quantize_fp8_block_ue8m0.restype = i32
    lib.dg_quantize_fp8_block_ue8m0.argtypes = [vp, vp, vp, i64, i64, i32, vp]
    lib.dg_fp8_gemm_nt_ue8m0.restype = i32
    lib.dg_fp8_gemm_nt_ue8m0.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp,
                                         ctypes.c_size_t, vp]
    lib.dg_fp8_gemm_nt_epilogue.restype = i32
    lib.dg_fp8_gemm_nt_epilogue.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i32, vp, vp,
                                            ctypes.c_size_t, vp]
    lib.dg_transpose_fp8.restype = i32
    lib.dg_transpose_fp8.argtypes = [vp, vp, i64, i64, vp]
    lib.dg_fp8_gemm_workspace_bytes.restype = ctypes.c_size_t
    lib.dg_fp8_gemm_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.dg_fp8_gemm.restype = i32
    lib.dg_fp8_gemm.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, i32, vp, ctypes.c_size_t,
                                vp]
    lib.dg_fp8_grouped_gemm_k.restype = i32
    lib.dg_fp8_grouped_gemm_k.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64, i64, i64, vp]
    lib.dg_fp8_gemm_nt_fused_a.restype = i32
    lib.dg_fp8_gemm_nt_fused_a.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, ctypes.c_size_t,
                                           vp]
    lib.dg_fp8_gemm_nt_fused_a_bf16.restype = i32
    lib.dg_fp8_gemm_nt_fused_a_bf16.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp,
                                                ctypes.c_size_t, vp]
    lib.dg_fp8_grouped_gemm_contig.restype = i32
    lib.dg_fp8_grouped_gemm_contig.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64, i64, i64, vp]
    lib.dg_fp8_grouped_gemm_masked_workspace_bytes.restype = ctypes.c_size_t
    lib.dg_fp8_grouped_gemm_masked_workspace_bytes.argtypes = [i32, i64, i64, i64]
    lib.dg_fp8_grouped_gemm_contig_epilogue.restype = i32
    lib.dg_fp8_grouped_gemm_contig_epilogue.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64, i64,
                                                        i64, i32, vp, vp]
    lib.dg_fp8_grouped_gemm_masked_epilogue.restype = i32
    lib.dg_fp8_grouped_gemm_masked_epilogue.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64, i64,
                                                        i64, i32, vp, vp, ctypes.c_size_t, vp]
    lib.dg_fp8_grouped_gemm_contig_workspace_bytes.restype = ctypes.c_size_t
    lib.dg_fp8_grouped_gemm_contig_workspace_bytes.argtypes = [i64, i64, i64]
    lib.dg_fp8_grouped_gemm_contig_balanced.restype = i32
    lib.dg_fp8_grouped_gemm_contig_balanced.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64, i64,
                                                        i64, i32, vp, vp, ctypes.c_size_t, vp]
    lib.dg_fp8_grouped_gemm_contig_ue8m0.restype = i32
    lib.dg_fp8_grouped_gemm_contig_ue8m0.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64, i64,
                                                     i64, vp]
    lib.dg_fp8_grouped_gemm_masked_ue8m0.restype = i32
    lib.dg_fp8_grouped_gemm_masked_ue8m0.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64, i64,
                                                     i64, vp, ctypes.c_size_t, vp]
    lib.dg_fp8_grouped_gemm_masked.restype = i32
    lib.dg_fp8_grouped_gemm_masked.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64, i64, i64, vp,
                                               ctypes.c_size_t, vp]
    lib.dg_fp8_gemm_nt_noalloc.restype = i32
    lib.dg_fp8_gemm_nt_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    if lib.dg_abi_version() != ABI_VERSION:
        raise ImportError("libdg ABI %d != binding ABI %d" % (lib.dg_abi_version(), ABI_VERSION))
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.dg_status_string(status).decode()


def get_mk_alignment_for_contiguous_layout() -> int:
    return lib.dg_get_mk_alignment_for_contiguous_layout()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream)


def _check(rc: int, where: str):
    if rc != DG_OK:
        raise DGError(rc, where)


def _require(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _codes(t, name):
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _require(t, torch.uint8, name)
    return t


def _bf16(t, name):
    if t.dtype in (torch.bfloat16, getattr(torch, "uint16", torch.int16)):
        t = t.view(torch.int16)
    _require(t, torch.int16, name)
    return t


def _workspace_bytes(workspace) -> int:
    if workspace is None:
        return 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace.numel() * workspace.element_size()


def alloc_workspace(nbytes: int, device="cuda"):
    """A split-K workspace of at least nbytes (16 minimum), zero-filled: its
    counter region must be zero before first use; every call leaves it zero,
    so the tensor can be reused by later calls ordered after this one."""
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


# ---------------------------------------------------------------------------
# C-ABI entry points
# ---------------------------------------------------------------------------

def dg_quantize_fp8_block(q, scales, x, block_rows: int = 128, stream=None) -> None:
    """x float32 [rows, cols] -> q (uint8/float8_e4m3fn [rows, cols]),
    scales float32 [ceil(cols/128), ceil(rows/block_rows)]."""
    _require(x, torch.float32, "x")
    q = _codes(q, "q")
    _require(scales, torch.float32, "scales")
    rows, cols = x.shape
    if q.shape != x.shape:
        raise ValueError("q must have the shape of x")
    if scales.numel() != cdiv(cols, 128) * cdiv(rows, block_rows):
        raise ValueError("scales must hold ceil(cols/128)*ceil(rows/block_rows) floats")
    _check(lib.dg_quantize_fp8_block(_ptr(q), _ptr(scales), _ptr(x), rows, cols, block_rows,
                                     _stream(stream)), "dg_quantize_fp8_block")


def dg_fp8_gemm_nt_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib.dg_fp8_gemm_nt_workspace_bytes(M, N, K)


def dg_fp8_gemm_nt(c, a, b, sa, sb, a_block_rows: int = 128, workspace=None,
                   stream=None) -> None:
    """C[M,N] (bf16) = block-scaled A[M,K] . B[N,K]^T."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sa, torch.float32, "sa")
    _require(sb, torch.float32, "sb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or c.shape != (M, N):
        raise ValueError("shape mismatch: a %s, b %s, c %s" % (tuple(a.shape), tuple(b.shape),
                                                              tuple(c.shape)))
    if sa.numel() != cdiv(K, 128) * cdiv(M, a_block_rows):
        raise ValueError("sa must hold (K/128)*ceil(M/a_block_rows) floats")
    if sb.numel() != cdiv(K, 128) * cdiv(N, 128):
        raise ValueError("sb must hold (K/128)*ceil(N/128) floats")
    ws_bytes = _workspace_bytes(workspace)
    _check(lib.dg_fp8_gemm_nt(_ptr(c), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), a_block_rows,
                              M, N, K, _ptr(workspace), ws_bytes, _stream(stream)),
           "dg_fp8_gemm_nt")


# static split-K scratch of dg_fp8_gemm_nt_noalloc, per GPU (dg.h)
NOALLOC_SCRATCH_BYTES = 16 << 20


def dg_fp8_gemm_nt_noalloc(c, a, b, sa, sb, a_block_rows: int = 128, stream=None) -> None:
    """dg_fp8_gemm_nt without a workspace argument, for callers that cannot
    allocate: the split-K scratch is the library's static per-GPU array
    (calls that overlap on one GPU race on it)."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sa, torch.float32, "sa")
    _require(sb, torch.float32, "sb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or c.shape != (M, N):
        raise ValueError("shape mismatch: a %s, b %s, c %s" % (tuple(a.shape), tuple(b.shape),
                                                              tuple(c.shape)))
    if sa.numel() != cdiv(K, 128) * cdiv(M, a_block_rows):
        raise ValueError("sa must hold (K/128)*ceil(M/a_block_rows) floats")
    if sb.numel() != cdiv(K, 128) * cdiv(N, 128):
        raise ValueError("sb must hold (K/128)*ceil(N/128) floats")
    _check(lib.dg_fp8_gemm_nt_noalloc(_ptr(c), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), a_block_rows,
                                      M, N, K, _stream(stream)), "dg_fp8_gemm_nt_noalloc")


def dg_quantize_fp8_block_ue8m0(q, sf, x, block_rows: int = 128, stream=None) -> None:
    """x float32 [rows, cols] -> q (uint8/float8_e4m3fn [rows, cols]),
    sf int32 [ceil(cols/512), ceil(rows/block_rows)] (UE8M0 exponents, four K
    blocks per word)."""
    _require(x, torch.float32, "x")
    q = _codes(q, "q")
    _require(sf, torch.int32, "sf")
    rows, cols = x.shape
    if q.shape != x.shape:
        raise ValueError("q must have the shape of x")
    if sf.numel() != cdiv(cdiv(cols, 128), 4) * cdiv(rows, block_rows):
        raise ValueError("sf must hold ceil(cols/512)*ceil(rows/block_rows) int32")
    _check(lib.dg_quantize_fp8_block_ue8m0(_ptr(q), _ptr(sf), _ptr(x), rows, cols, block_rows,
                                           _stream(stream)), "dg_quantize_fp8_block_ue8m0")


def dg_fp8_gemm_nt_ue8m0(c, a, b, sfa, sfb, a_block_rows: int = 128, workspace=None,
                         stream=None) -> None:
    """C[M,N] (bf16) = A[M,K] . B[N,K]^T with packed UE8M0 block scales."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sfa, torch.int32, "sfa")
    _require(sfb, torch.int32, "sfb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or c.shape != (M, N):
        raise ValueError("shape mismatch: a %s, b %s, c %s" % (tuple(a.shape), tuple(b.shape),
                                                              tuple(c.shape)))
    if sfa.numel() != cdiv(cdiv(K, 128), 4) * cdiv(M, a_block_rows):
        raise ValueError("sfa must hold ceil(K/512)*ceil(M/a_block_rows) int32")
    if sfb.numel() != cdiv(cdiv(K, 128), 4) * cdiv(N, 128):
        raise ValueError("sfb must hold ceil(K/512)*ceil(N/128) int32")
    _check(lib.dg_fp8_gemm_nt_ue8m0(_ptr(c), _ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb), a_block_rows,
                                    M, N, K, _ptr(workspace), _workspace_bytes(workspace),
                                    _stream(stream)), "dg_fp8_gemm_nt_ue8m0")


FUSED_A_MAX_M = 64


def dg_fp8_gemm_nt_fused_a(c, a, b, sb, workspace=None, stream=None) -> None:
    """C[M,N] (bf16) = A[M,K] (float32 or bfloat16, quantised with 1x128
    blocks inside the GEMM) . B[N,K]^T (E4M3, 128x128 scales sb);
    M <= FUSED_A_MAX_M."""
    c = _bf16(c, "c")
    if not isinstance(a, torch.Tensor) or a.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("a must be a float32 or bfloat16 tensor")
    bf16 = a.dtype == torch.bfloat16
    _require(a, a.dtype, "a")
    b = _codes(b, "b")
    _require(sb, torch.float32, "sb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K or c.shape != (M, N):
        raise ValueError("shape mismatch: a %s, b %s, c %s" % (tuple(a.shape), tuple(b.shape),
                                                              tuple(c.shape)))
    if sb.numel() != cdiv(K, 128) * cdiv(N, 128):
        raise ValueError("sb must hold (K/128)*ceil(N/128) floats")
    ws_bytes = _workspace_bytes(workspace)
    fn = lib.dg_fp8_gemm_nt_fused_a_bf16 if bf16 else lib.dg_fp8_gemm_nt_fused_a
    _check(fn(_ptr(c), _ptr(a), _ptr(b), _ptr(sb), M, N, K, _ptr(workspace), ws_bytes,
              _stream(stream)), "dg_fp8_gemm_nt_fused_a" + ("_bf16" if bf16 else ""))


EPILOGUES = {"none": 0, "relu": 1, "silu": 2, "gelu": 3, "swiglu": 4}


def dg_fp8_gemm_nt_epilogue(c, a, b, sa, sb, a_block_rows: int = 128, act: str = "none",
                            residual=None, workspace=None, stream=None) -> None:
    """C = epilogue(A . B^T): act in EPILOGUES (swiglu: B rows interleave gate
    and up, C has N/2 columns), plus an optional BF16 residual [M, Nout]
    (may be c itself)."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sa, torch.float32, "sa")
    _require(sb, torch.float32, "sb")
    M, K = a.shape
    N = b.shape[0]
    code = EPILOGUES[act]
    n_out = N // 2 if code == EPILOGUES["swiglu"] else N
    if b.shape[1] != K or c.shape != (M, n_out):
        raise ValueError("shape mismatch: a %s, b %s, c %s (act %s)"
                         % (tuple(a.shape), tuple(b.shape), tuple(c.shape), act))
    if sa.numel() != cdiv(K, 128) * cdiv(M, a_block_rows):
        raise ValueError("sa must hold (K/128)*ceil(M/a_block_rows) floats")
    if sb.numel() != cdiv(K, 128) * cdiv(N, 128):
        raise ValueError("sb must hold (K/128)*ceil(N/128) floats")
    if residual is not None:
        residual = _bf16(residual, "residual")
        if residual.shape != (M, n_out):
            raise ValueError("residual must be [M, Nout]")
    _check(lib.dg_fp8_gemm_nt_epilogue(_ptr(c), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), a_block_rows,
                                       M, N, K, code, _ptr(residual), _ptr(workspace),
                                       _workspace_bytes(workspace), _stream(stream)),
           "dg_fp8_gemm_nt_epilogue")


LAYOUTS = {"nt": 0, "tn": 1, "nn": 2, "tt": 3}


def dg_transpose_fp8(out, inp, stream=None) -> None:
    """out [cols, rows] = inp [rows, cols]^T (bytes; rows, cols multiples of 16)."""
    out = _codes(out, "out")
    inp = _codes(inp, "inp")
    rows, cols = inp.shape
    if out.shape != (cols, rows):
        raise ValueError("out must be [cols, rows]")
    _check(lib.dg_transpose_fp8(_ptr(out), _ptr(inp), rows, cols, _stream(stream)),
           "dg_transpose_fp8")


def dg_fp8_gemm_workspace_bytes(M: int, N: int, K: int, layout: str = "nt") -> int:
    return lib.dg_fp8_gemm_workspace_bytes(M, N, K, LAYOUTS[layout])


def dg_fp8_gemm(c, a, b, sa, sb, a_block_rows: int = 128, layout: str = "nt", workspace=None,
                stream=None) -> None:
    """C[M,N] = A . B^T with operands stored per ``layout`` (first letter A:
    n = [M,K], t = [K,M]; second letter B: t = [N,K], n = [K,N])."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sa, torch.float32, "sa")
    _require(sb, torch.float32, "sb")
    M, N = c.shape
    a_t = layout in ("tn", "tt")
    b_n = layout in ("tn", "nn")
    K = a.shape[0] if a_t else a.shape[1]
    if a.shape != ((K, M) if a_t else (M, K)) or b.shape != ((K, N) if b_n else (N, K)):
        raise ValueError("shape mismatch for layout %s: a %s, b %s, c %s"
                         % (layout, tuple(a.shape), tuple(b.shape), tuple(c.shape)))
    if sa.numel() != cdiv(K, 128) * cdiv(M, a_block_rows):
        raise ValueError("sa must hold (K/128)*ceil(M/a_block_rows) floats")
    if sb.numel() != cdiv(K, 128) * cdiv(N, 128):
        raise ValueError("sb must hold (K/128)*ceil(N/128) floats")
    _check(lib.dg_fp8_gemm(_ptr(c), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), a_block_rows, M, N, K,
                           LAYOUTS[layout], _ptr(workspace), _workspace_bytes(workspace),
                           _stream(stream)), "dg_fp8_gemm")


def dg_fp8_grouped_gemm_k(c, a, b, sa, sb, a_block_rows: int, k_offsets, stream=None) -> None:
    """K-grouped: c [G, M, N] (bf16), a [M, K], b [N, K], k_offsets int64
    device [G + 1] (multiples of 128): c[g] = A[:, k0:k1] . B[:, k0:k1]^T."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sa, torch.float32, "sa")
    _require(sb, torch.float32, "sb")
    _require(k_offsets, torch.int64, "k_offsets")
    M, K = a.shape
    N = b.shape[0]
    G = k_offsets.numel() - 1
    if b.shape[1] != K or c.shape != (G, M, N):
        raise ValueError("shape mismatch")
    if sa.numel() != cdiv(K, 128) * cdiv(M, a_block_rows):
        raise ValueError("sa must hold (K/128)*ceil(M/a_block_rows) floats")
    if sb.numel() != cdiv(K, 128) * cdiv(N, 128):
        raise ValueError("sb must hold (K/128)*ceil(N/128) floats")
    _check(lib.dg_fp8_grouped_gemm_k(_ptr(c), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb), a_block_rows,
                                     _ptr(k_offsets), G, M, N, K, _stream(stream)),
           "dg_fp8_grouped_gemm_k")


def dg_fp8_grouped_gemm_contig_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib.dg_fp8_grouped_gemm_contig_workspace_bytes(M, N, K)


def dg_fp8_grouped_gemm_contig(c, a, b, sa, sb, a_block_rows: int, m_indices, act: str = "none",
                               residual=None, workspace=None, stream=None) -> None:
    """Grouped M-contiguous: a [M,K], b [G,N,K], sb [G,K/128,ceil(N/128)],
    m_indices int32 [M] (-1 = padding row -> zero row).  act / residual: the
    fused epilogue (swiglu: each expert's B rows interleave gate and up, c has
    N/2 columns); padding rows stay zero.  workspace (zero-filled device
    bytes, dg_fp8_grouped_gemm_contig_workspace_bytes(M, N, K) of them; see
    alloc_workspace): share the work evenly over the compute units
    (dg_fp8_grouped_gemm_contig_balanced)."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sa, torch.float32, "sa")
    _require(sb, torch.float32, "sb")
    _require(m_indices, torch.int32, "m_indices")
    M, K = a.shape
    G, N, Kb = b.shape
    code = EPILOGUES[act]
    n_out = N // 2 if code == EPILOGUES["swiglu"] else N
    if Kb != K or c.shape != (M, n_out) or m_indices.shape != (M,):
        raise ValueError("inconsistent grouped GEMM shapes")
    if sa.numel() != cdiv(K, 128) * cdiv(M, a_block_rows):
        raise ValueError("sa must hold (K/128)*ceil(M/a_block_rows) floats")
    if sb.numel() != G * cdiv(K, 128) * cdiv(N, 128):
        raise ValueError("sb must hold G*(K/128)*ceil(N/128) floats")
    if residual is not None:
        residual = _bf16(residual, "residual")
        if residual.shape != (M, n_out):
            raise ValueError("residual must be [M, Nout]")
    if workspace is not None:
        rc = lib.dg_fp8_grouped_gemm_contig_balanced(_ptr(c), _ptr(a), _ptr(b), _ptr(sa),
                                                     _ptr(sb), a_block_rows, _ptr(m_indices), G,
                                                     M, N, K, code, _ptr(residual),
                                                     _ptr(workspace), _workspace_bytes(workspace),
                                                     _stream(stream))
    elif code == 0 and residual is None:
        rc = lib.dg_fp8_grouped_gemm_contig(_ptr(c), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb),
                                            a_block_rows, _ptr(m_indices), G, M, N, K,
                                            _stream(stream))
    else:
        rc = lib.dg_fp8_grouped_gemm_contig_epilogue(_ptr(c), _ptr(a), _ptr(b), _ptr(sa),
                                                     _ptr(sb), a_block_rows, _ptr(m_indices), G,
                                                     M, N, K, code, _ptr(residual),
                                                     _stream(stream))
    _check(rc, "dg_fp8_grouped_gemm_contig")


def dg_fp8_grouped_gemm_contig_ue8m0(c, a, b, sfa, sfb, a_block_rows: int, m_indices,
                                     stream=None) -> None:
    """Grouped M-contiguous with packed UE8M0 scales: sfa int32
    [ceil(K/512), ceil(M/br)], sfb int32 [G, ceil(K/512), ceil(N/128)]."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sfa, torch.int32, "sfa")
    _require(sfb, torch.int32, "sfb")
    _require(m_indices, torch.int32, "m_indices")
    M, K = a.shape
    G, N, Kb = b.shape
    if Kb != K or c.shape != (M, N) or m_indices.shape != (M,):
        raise ValueError("inconsistent grouped GEMM shapes")
    if sfa.numel() != cdiv(cdiv(K, 128), 4) * cdiv(M, a_block_rows):
        raise ValueError("sfa must hold ceil(K/512)*ceil(M/a_block_rows) int32")
    if sfb.numel() != G * cdiv(cdiv(K, 128), 4) * cdiv(N, 128):
        raise ValueError("sfb must hold G*ceil(K/512)*ceil(N/128) int32")
    _check(lib.dg_fp8_grouped_gemm_contig_ue8m0(_ptr(c), _ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb),
                                                a_block_rows, _ptr(m_indices), G, M, N, K,
                                                _stream(stream)), "dg_fp8_grouped_gemm_contig_ue8m0")


def dg_fp8_grouped_gemm_masked_ue8m0(c, a, b, sfa, sfb, a_block_rows: int, masked_m,
                                     workspace=None, stream=None) -> None:
    """Masked grouped with packed UE8M0 scales: sfa int32
    [G, ceil(K/512), ceil(max_m/br)], sfb int32 [G, ceil(K/512), ceil(N/128)]."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sfa, torch.int32, "sfa")
    _require(sfb, torch.int32, "sfb")
    _require(masked_m, torch.int32, "masked_m")
    G, max_m, K = a.shape
    Gb, N, Kb = b.shape
    if Gb != G or Kb != K or c.shape != (G, max_m, N) or masked_m.shape != (G,):
        raise ValueError("inconsistent masked grouped GEMM shapes")
    if sfa.numel() != G * cdiv(cdiv(K, 128), 4) * cdiv(max_m, a_block_rows):
        raise ValueError("sfa must hold G*ceil(K/512)*ceil(max_m/a_block_rows) int32")
    if sfb.numel() != G * cdiv(cdiv(K, 128), 4) * cdiv(N, 128):
        raise ValueError("sfb must hold G*ceil(K/512)*ceil(N/128) int32")
    _check(lib.dg_fp8_grouped_gemm_masked_ue8m0(_ptr(c), _ptr(a), _ptr(b), _ptr(sfa), _ptr(sfb),
                                                a_block_rows, _ptr(masked_m), G, max_m, N, K,
                                                _ptr(workspace), _workspace_bytes(workspace),
                                                _stream(stream)), "dg_fp8_grouped_gemm_masked_ue8m0")


def dg_fp8_grouped_gemm_masked_workspace_bytes(num_groups: int, max_m: int, N: int,
                                              K: int) -> int:
    return lib.dg_fp8_grouped_gemm_masked_workspace_bytes(num_groups, max_m, N, K)


def dg_fp8_grouped_gemm_masked(c, a, b, sa, sb, a_block_rows: int, masked_m, workspace=None,
                               act: str = "none", residual=None, stream=None) -> None:
    """Masked grouped: a [G,max_m,K], b [G,N,K], sa [G,K/128,ceil(max_m/br)],
    sb [G,K/128,ceil(N/128)], masked_m int32 [G] (device), c [G,max_m,Nout]
    (Nout = N, or N/2 with act="swiglu"); rows past masked_m[g] of c[g] are
    not written.  act / residual [G,max_m,Nout]: the fused epilogue."""
    c = _bf16(c, "c")
    a = _codes(a, "a")
    b = _codes(b, "b")
    _require(sa, torch.float32, "sa")
    _require(sb, torch.float32, "sb")
    _require(masked_m, torch.int32, "masked_m")
    G, max_m, K = a.shape
    Gb, N, Kb = b.shape
    code = EPILOGUES[act]
    n_out = N // 2 if code == EPILOGUES["swiglu"] else N
    if Gb != G or Kb != K or c.shape != (G, max_m, n_out) or masked_m.shape != (G,):
        raise ValueError("inconsistent masked grouped GEMM shapes")
    if sa.numel() != G * cdiv(K, 128) * cdiv(max_m, a_block_rows):
        raise ValueError("sa must hold G*(K/128)*ceil(max_m/a_block_rows) floats")
    if sb.numel() != G * cdiv(K, 128) * cdiv(N, 128):
        raise ValueError("sb must hold G*(K/128)*ceil(N/128) floats")
    if residual is not None:
        residual = _bf16(residual, "residual")
        if residual.shape != (G, max_m, n_out):
            raise ValueError("residual must be [G, max_m, Nout]")
    if code == 0 and residual is None:
        rc = lib.dg_fp8_grouped_gemm_masked(_ptr(c), _ptr(a), _ptr(b), _ptr(sa), _ptr(sb),
                                            a_block_rows, _ptr(masked_m), G, max_m, N, K,
                                            _ptr(workspace), _workspace_bytes(workspace),
                                            _stream(stream))
    else:
        rc = lib.dg_fp8_grouped_gemm_masked_epilogue(_ptr(c), _ptr(a), _ptr(b), _ptr(sa),
                                                     _ptr(sb), a_block_rows, _ptr(masked_m), G,
                                                     max_m, N, K, code, _ptr(residual),
                                                     _ptr(workspace), _workspace_bytes(workspace),
                                                     _stream(stream))
    _check(rc, "dg_fp8_grouped_gemm_masked")


# ---------------------------------------------------------------------------
# Conveniences (allocate outputs with torch)
# ---------------------------------------------------------------------------

def to_fp8(x, block_rows: int = 128):
    """Quantise a float32 device matrix -> (codes uint8 [R, C], scales float32
    [ceil(C/128), ceil(R/block_rows)])."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((cdiv(cols, 128), cdiv(rows, block_rows)), dtype=torch.float32,
                    device=x.device)
    dg_quantize_fp8_block(q, s, x, block_rows)
    return q, s


def to_fp8_ue8m0(x, block_rows: int = 128):
    """Quantise with power-of-two scales -> (codes uint8 [R, C], packed UE8M0
    exponents int32 [ceil(C/512), ceil(R/block_rows)])."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    sf = torch.empty((cdiv(cdiv(cols, 128), 4), cdiv(rows, block_rows)), dtype=torch.int32,
                     device=x.device)
    dg_quantize_fp8_block_ue8m0(q, sf, x, block_rows)
    return q, sf


def fp8_gemm_nt(c, a, b, sa, sb, a_block_rows: int = 128, workspace=None):
    dg_fp8_gemm_nt(c, a, b, sa, sb, a_block_rows, workspace)
    return c


def fp8_grouped_gemm_contig(c, a, b, sa, sb, m_indices, a_block_rows: int = 1):
    dg_fp8_grouped_gemm_contig(c, a, b, sa, sb, a_block_rows, m_indices, workspace=None)
    return c


__all__ = [
    "lib", "LIB_PATH", "DGError", "status_string", "get_mk_alignment_for_contiguous_layout",
    "dg_quantize_fp8_block", "dg_fp8_gemm_nt_workspace_bytes", "dg_fp8_gemm_nt",
    "dg_fp8_gemm_nt_fused_a", "FUSED_A_MAX_M", "dg_fp8_grouped_gemm_contig", "to_fp8",
    "dg_quantize_fp8_block_ue8m0", "dg_fp8_gemm_nt_ue8m0", "to_fp8_ue8m0",
    "dg_fp8_gemm_nt_epilogue", "EPILOGUES", "dg_transpose_fp8", "dg_fp8_gemm_workspace_bytes",
    "dg_fp8_gemm", "LAYOUTS", "dg_fp8_grouped_gemm_k", "fp8_gemm_nt", "fp8_grouped_gemm_contig",
    "dg_fp8_grouped_gemm_masked", "dg_fp8_grouped_gemm_masked_workspace_bytes",
    "dg_fp8_grouped_gemm_contig_ue8m0", "dg_fp8_grouped_gemm_masked_ue8m0", "alloc_workspace",
    "WORKSPACE_COUNTER_BYTES", "dg_fp8_gemm_nt_noalloc", "NOALLOC_SCRATCH_BYTES",
]
# (the _epilogue C entry points are reached through the act / residual
# arguments of dg_fp8_grouped_gemm_contig and dg_fp8_grouped_gemm_masked)
