"""CPU oracle for FP8 E4M3 block-scaled quantisation and the dequantised NT GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``fp8_block_scaled_dg_amd``) never imports, links or runs it, and it
shares no code with the HIP kernels.

The arithmetic lives in ``oracle.c`` (plain C, FP64 accumulation); this module
only marshals numpy arrays through ctypes.  Every function cites the passage it
follows in ``oracle.c`` / ``oracle.h``:

* "DeepGEMM ... FP8 block-quantised GEMM" (lpnh.cn/news/2826317) s2.2, s3.1,
  s3.2, s4.2, s5.4 -- block scaling, scale = max_abs/448, RNE to E4M3, FP32
  accumulation of dequantised products.
* "DeepGEMM: GPU high-efficiency BLAS kernel library" (pzsr.cn/news/21800)
  s3.1-s3.3, s4.1 -- NT layout, FP32 scales, grouped contiguous layout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no fast-math, no FP contraction)."""
    stale = (not os.path.exists(_LIB)) or any(
        os.path.getmtime(p) > os.path.getmtime(_LIB) for p in (_SRC, _HDR))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64 = ctypes.c_int64
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode_arith.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_arith.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode_search.restype = ctypes.c_uint8
    lib.orc_e4m3_encode_search.argtypes = [ctypes.c_float]
    for name in ("orc_e4m3_encode_arith_n", "orc_e4m3_encode_search_n"):
        fn = getattr(lib, name)
        fn.restype = None
        fn.argtypes = [f32p, u8p, i64]
    lib.orc_e4m3_decode_n.restype = None
    lib.orc_e4m3_decode_n.argtypes = [u8p, f64p, i64]
    lib.orc_quantize_block.restype = ctypes.c_int
    lib.orc_quantize_block.argtypes = [f32p, i64, i64, ctypes.c_int, u8p, f32p]
    lib.orc_quantize_block_ue8m0.restype = ctypes.c_int
    lib.orc_quantize_block_ue8m0.argtypes = [f32p, i64, i64, ctypes.c_int, u8p, u8p]
    lib.orc_ue8m0_pack.restype = None
    lib.orc_ue8m0_pack.argtypes = [u8p, i64, i64, ctypes.POINTER(ctypes.c_uint32)]
    lib.orc_grouped_gemm_k.restype = ctypes.c_int
    lib.orc_grouped_gemm_k.argtypes = [u8p, f32p, ctypes.c_int, u8p, f32p, i64p, ctypes.c_int,
                                       i64, i64, i64, f64p]
    lib.orc_epilogue.restype = ctypes.c_int
    lib.orc_epilogue.argtypes = [f64p, i64, i64, ctypes.c_int, ctypes.POINTER(ctypes.c_uint16),
                                 f64p]
    lib.orc_quantize_global.restype = ctypes.c_int
    lib.orc_quantize_global.argtypes = [f32p, i64, i64, u8p, f32p]
    lib.orc_gemm_nt.restype = ctypes.c_int
    lib.orc_gemm_nt.argtypes = [u8p, f32p, ctypes.c_int, u8p, f32p, i64, i64, i64, f64p]
    lib.orc_gemm_nt_points.restype = ctypes.c_int
    lib.orc_gemm_nt_points.argtypes = [u8p, f32p, ctypes.c_int, u8p, f32p, i64, i64, i64,
                                       i64p, i64p, i64, f64p]
    lib.orc_grouped_gemm_contig.restype = ctypes.c_int
    lib.orc_grouped_gemm_contig.argtypes = [u8p, f32p, ctypes.c_int, u8p, f32p, i32p,
                                            ctypes.c_int, i64, i64, i64, i64, i64, f64p]
    lib.orc_grouped_gemm_masked.restype = ctypes.c_int
    lib.orc_grouped_gemm_masked.argtypes = [u8p, f32p, ctypes.c_int, u8p, f32p, i32p,
                                            ctypes.c_int, i64, i64, i64, f64p]
    _lib = lib
    return lib


def _ptr(arr: np.ndarray, ctype):
    return arr.ctypes.data_as(ctypes.POINTER(ctype))


def _c(arr, dtype) -> np.ndarray:
    return np.ascontiguousarray(arr, dtype=dtype)


def cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


# --------------------------------------------------------------------------
# Codec
# --------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """E4M3 code bytes -> float64 values (NaN for S.1111.111)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_e4m3_decode_n(_ptr(c, ctypes.c_uint8), _ptr(out, ctypes.c_double), c.size)
    return out


def e4m3_encode(values, method: str = "arith") -> np.ndarray:
    """float32 values -> E4M3 codes, round-to-nearest-even, saturating, sign kept."""
    v = _c(values, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    fn = {"arith": _load().orc_e4m3_encode_arith_n,
          "search": _load().orc_e4m3_encode_search_n}[method]
    fn(_ptr(v, ctypes.c_float), _ptr(out, ctypes.c_uint8), v.size)
    return out


# --------------------------------------------------------------------------
# Quantiser and GEMMs
# --------------------------------------------------------------------------

def quantize(x, block_rows: int = 128):
    """x: float32 [rows, cols] -> (q uint8 [rows, cols],
    scales float32 [ceil(cols/128), ceil(rows/block_rows)])."""
    x = _c(x, np.float32)
    assert x.ndim == 2
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((cdiv(cols, 128), cdiv(rows, block_rows)), dtype=np.float32)
    rc = _load().orc_quantize_block(_ptr(x, ctypes.c_float), rows, cols, block_rows,
                                    _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle quantize rejected its input")
    return q, s


def quantize_global(x):
    """x: float32 [rows, cols] -> (q uint8 [rows, cols], scale float) with one
    scale for the whole tensor (bjdmk.com.cn DeepGEMM page s3.3 contrasts this
    with per-block scales)."""
    x = _c(x, np.float32)
    assert x.ndim == 2
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty(1, dtype=np.float32)
    rc = _load().orc_quantize_global(_ptr(x, ctypes.c_float), rows, cols,
                                     _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle quantize_global rejected its input")
    return q, float(s[0])


def quantize_ue8m0(x, block_rows: int = 128):
    """Block quantiser with power-of-two scales (pzsr.cn DeepGEMM page s3.1,
    UE8M0; the power of two is binary32(amax/448) rounded up -- see oracle.c).
    x: float32 [rows, cols] -> (q uint8 [rows, cols],
    exps uint8 [ceil(cols/128), ceil(rows/block_rows)], scale = 2^(E-127))."""
    x = _c(x, np.float32)
    assert x.ndim == 2
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.uint8)
    e = np.empty((cdiv(cols, 128), cdiv(rows, block_rows)), dtype=np.uint8)
    rc = _load().orc_quantize_block_ue8m0(_ptr(x, ctypes.c_float), rows, cols, block_rows,
                                          _ptr(q, ctypes.c_uint8), _ptr(e, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("oracle quantize_ue8m0 rejected its input")
    return q, e


def pack_ue8m0(exps) -> np.ndarray:
    """uint8 [n_kb, n_rb] -> int32 [ceil(n_kb/4), n_rb], four exponents per word
    along K blocks (byte kb % 4, least significant first; unused bytes 0)."""
    e = _c(exps, np.uint8)
    n_kb, n_rb = e.shape
    out = np.empty((cdiv(n_kb, 4), n_rb), dtype=np.uint32)
    _load().orc_ue8m0_pack(_ptr(e, ctypes.c_uint8), n_kb, n_rb, _ptr(out, ctypes.c_uint32))
    return out.view(np.int32)


def ue8m0_scales(exps) -> np.ndarray:
    """Exponents -> float32 scales 2^(E-127) (exact: 2^-127 is a binary32
    subnormal), for use with gemm_nt / gemm_nt_points."""
    e = np.asarray(exps, dtype=np.int64)
    return np.ldexp(np.float32(1.0), (e - 127).astype(np.int32)).astype(np.float32)


def _check_gemm(qa, sa, a_block_rows, qb, sb):
    qa = _c(qa, np.uint8)
    qb = _c(qb, np.uint8)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    M, K = qa.shape
    N = qb.shape[-2]
    assert qb.shape[-1] == K
    assert sa.shape == (cdiv(K, 128), cdiv(M, a_block_rows)), (sa.shape, M, K)
    return qa, sa, qb, sb, M, N, K


def gemm_nt(qa, sa, qb, sb, a_block_rows: int = 128) -> np.ndarray:
    """Dequantised C = A . B^T in float64, [M, N]."""
    qa, sa, qb, sb, M, N, K = _check_gemm(qa, sa, a_block_rows, qb, sb)
    assert sb.shape == (cdiv(K, 128), cdiv(N, 128))
    ref = np.empty((M, N), dtype=np.float64)
    rc = _load().orc_gemm_nt(_ptr(qa, ctypes.c_uint8), _ptr(sa, ctypes.c_float), a_block_rows,
                             _ptr(qb, ctypes.c_uint8), _ptr(sb, ctypes.c_float), M, N, K,
                             _ptr(ref, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle gemm_nt rejected its input")
    return ref


def gemm_nt_points(qa, sa, qb, sb, pm, pn, a_block_rows: int = 128) -> np.ndarray:
    """The same product at the positions (pm[i], pn[i]) only."""
    qa, sa, qb, sb, M, N, K = _check_gemm(qa, sa, a_block_rows, qb, sb)
    assert sb.shape == (cdiv(K, 128), cdiv(N, 128))
    pm = _c(pm, np.int64)
    pn = _c(pn, np.int64)
    assert pm.shape == pn.shape
    out = np.empty(pm.shape, dtype=np.float64)
    rc = _load().orc_gemm_nt_points(_ptr(qa, ctypes.c_uint8), _ptr(sa, ctypes.c_float),
                                    a_block_rows, _ptr(qb, ctypes.c_uint8),
                                    _ptr(sb, ctypes.c_float), M, N, K,
                                    _ptr(pm, ctypes.c_int64), _ptr(pn, ctypes.c_int64),
                                    pm.size, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle gemm_nt_points rejected its input")
    return out


def grouped_gemm_contig(qa, sa, qb, sb, m_indices, a_block_rows: int = 128,
                        rows=None) -> np.ndarray:
    """Grouped M-contiguous product.  qb [G, N, K], sb [G, ceil(K/128), ceil(N/128)],
    m_indices int32 [M] (expert id, -1 = padding row -> zero output row).
    ``rows`` = (begin, end) restricts the rows computed; others are NaN."""
    qa, sa, qb, sb, M, N, K = _check_gemm(qa, sa, a_block_rows, qb, sb)
    G = qb.shape[0]
    assert qb.shape == (G, N, K)
    assert sb.shape == (G, cdiv(K, 128), cdiv(N, 128))
    mi = _c(m_indices, np.int32)
    assert mi.shape == (M,)
    r0, r1 = (0, M) if rows is None else rows
    ref = np.full((M, N), np.nan, dtype=np.float64)
    rc = _load().orc_grouped_gemm_contig(_ptr(qa, ctypes.c_uint8), _ptr(sa, ctypes.c_float),
                                         a_block_rows, _ptr(qb, ctypes.c_uint8),
                                         _ptr(sb, ctypes.c_float), _ptr(mi, ctypes.c_int32),
                                         G, M, N, K, r0, r1, _ptr(ref, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle grouped_gemm_contig rejected its input")
    return ref


def grouped_gemm_masked(qa, sa, qb, sb, masked_m, a_block_rows: int = 1) -> np.ndarray:
    """Masked grouped product (pzsr.cn DeepGEMM page s2.3, s3.2: expert
    weights batched in one call; the decode-time layout with a fixed capacity
    of max_m rows per expert, masked_m[g] of them valid).
    qa [G, max_m, K], sa [G, ceil(K/128), ceil(max_m/br)], qb [G, N, K],
    sb [G, ceil(K/128), ceil(N/128)], masked_m int32 [G] in [0, max_m].
    Returns float64 [G, max_m, N]; rows past masked_m[g] are NaN."""
    qa, qb = _c(qa, np.uint8), _c(qb, np.uint8)
    sa, sb = _c(sa, np.float32), _c(sb, np.float32)
    G, max_m, K = qa.shape
    N = qb.shape[1]
    assert qb.shape == (G, N, K)
    assert sa.shape == (G, cdiv(K, 128), cdiv(max_m, a_block_rows))
    assert sb.shape == (G, cdiv(K, 128), cdiv(N, 128))
    mm = _c(masked_m, np.int32)
    assert mm.shape == (G,)
    ref = np.full((G, max_m, N), np.nan, dtype=np.float64)
    rc = _load().orc_grouped_gemm_masked(_ptr(qa, ctypes.c_uint8), _ptr(sa, ctypes.c_float),
                                         a_block_rows, _ptr(qb, ctypes.c_uint8),
                                         _ptr(sb, ctypes.c_float), _ptr(mm, ctypes.c_int32),
                                         G, max_m, N, K, _ptr(ref, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle grouped_gemm_masked rejected its input")
    return ref


def grouped_gemm_k(qa, sa, qb, sb, k_offsets, a_block_rows: int = 1) -> np.ndarray:
    """K-grouped product (pzsr.cn DeepGEMM page s3.2, grouping along K for
    MoE weight gradients): out[g] = A[:, k0:k1] . B[:, k0:k1]^T with
    (k0, k1) = (k_offsets[g], k_offsets[g+1]), multiples of 128.
    qa [M, K], qb [N, K]; sa [K/128, ceil(M/br)], sb [K/128, ceil(N/128)].
    Returns float64 [G, M, N]."""
    qa, sa, qb, sb, M, N, K = _check_gemm(qa, sa, a_block_rows, qb, sb)
    assert sb.shape == (cdiv(K, 128), cdiv(N, 128))
    ko = _c(k_offsets, np.int64)
    G = ko.size - 1
    out = np.empty((G, M, N), dtype=np.float64)
    rc = _load().orc_grouped_gemm_k(_ptr(qa, ctypes.c_uint8), _ptr(sa, ctypes.c_float),
                                    a_block_rows, _ptr(qb, ctypes.c_uint8),
                                    _ptr(sb, ctypes.c_float), _ptr(ko, ctypes.c_int64), G, M, N, K,
                                    _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle grouped_gemm_k rejected its input")
    return out


EPILOGUES = {"none": 0, "relu": 1, "silu": 2, "gelu": 3, "swiglu": 4}


def epilogue(acc, act: str = "none", residual=None) -> np.ndarray:
    """Epilogue on a float64 product [M, N] (bjdmk.com.cn DeepGEMM page s3.2;
    SwiGLU per the pzsr.cn page s2.3): activation, or SwiGLU over interleaved
    gate/up columns (output N/2 columns), then + residual (BF16 bits as uint16
    [M, Nout]) if given.  Returns float64 [M, Nout]."""
    a = _c(acc, np.float64)
    M, N = a.shape
    code = EPILOGUES[act]
    n_out = N // 2 if code == 4 else N
    out = np.empty((M, n_out), dtype=np.float64)
    r = None
    if residual is not None:
        r = _c(residual, np.uint16)
        assert r.shape == (M, n_out)
    rc = _load().orc_epilogue(_ptr(a, ctypes.c_double), M, N, code,
                              None if r is None else _ptr(r, ctypes.c_uint16),
                              _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle epilogue rejected its input")
    return out
