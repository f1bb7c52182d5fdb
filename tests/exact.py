"""Exact-rational brute force used to pin the oracle.

Independent of ``oracle/``: the E4M3 value set is enumerated from the format's
field definition as exact fractions, rounding is a nearest search with exact
distances (ties to the even code), binary32 divisions are done by numpy's IEEE
float32 division, and decoding for the dequantised products uses PyTorch's
``float8_e4m3fn`` dtype.  Slow on purpose; used on tiny inputs only.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def _e4m3_magnitudes():
    vals = []
    for code in range(127):                       # 0x00 .. 0x7E, all finite
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(Fraction(m, 8) / 64)      # 2^-6 * m/8
        else:
            vals.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


E4M3_MAG = _e4m3_magnitudes()


def nearest_even_code(value: Fraction, negative: bool) -> int:
    """Nearest finite E4M3 magnitude to |value| (exact distances), ties to
    the even code; values beyond 448 land on 448 because it is the nearest
    finite magnitude."""
    a = abs(value)
    best = min(range(127), key=lambda c: (abs(a - E4M3_MAG[c]), c & 1))
    return best | (0x80 if negative else 0)


def f32(x) -> np.float32:
    return np.float32(x)


def torch_decode(codes) -> np.ndarray:
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def quantize_exact(x: np.ndarray, block_rows: int):
    """Brute-force block quantiser: amax by exact comparison, scale and
    quotient by numpy float32 division, nearest-even search over fractions."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    n_rb = -(-rows // block_rows)
    n_kb = -(-cols // 128)
    q = np.zeros((rows, cols), dtype=np.uint8)
    s = np.zeros((n_kb, n_rb), dtype=np.float32)
    for rb in range(n_rb):
        rsl = slice(rb * block_rows, min(rows, (rb + 1) * block_rows))
        for kb in range(n_kb):
            ksl = slice(kb * 128, min(cols, (kb + 1) * 128))
            blk = x[rsl, ksl]
            amax = max((abs(float(v)) for v in blk.ravel()), default=0.0)
            scale = np.float32(amax) / np.float32(448.0)
            s[kb, rb] = scale
            for i in range(blk.shape[0]):
                for j in range(blk.shape[1]):
                    xv = blk[i, j]
                    neg = bool(np.signbit(xv))
                    if scale == 0:
                        code = 0x80 if neg else 0
                    else:
                        v = np.float32(xv) / scale
                        code = nearest_even_code(Fraction(float(v)), neg)
                    q[rsl.start + i, ksl.start + j] = code
    return q, s


def gemm_exact(qa, sa, qb, sb, a_block_rows: int):
    """Exact rational value of sum_kb sa*sb*sum_k dec(qa)dec(qb), as a list of
    lists of Fractions."""
    da = torch_decode(qa)
    db = torch_decode(qb)
    M, K = da.shape
    N = db.shape[0]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            tot = Fraction(0)
            for kb in range(-(-K // 128)):
                ks = range(kb * 128, min(K, (kb + 1) * 128))
                p = sum((Fraction(float(da[m, k])) * Fraction(float(db[n, k])) for k in ks),
                        Fraction(0))
                tot += (Fraction(float(sa[kb, m // a_block_rows]))
                        * Fraction(float(sb[kb, n // 128])) * p)
            row.append(tot)
        out.append(row)
    return out
