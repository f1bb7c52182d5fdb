"""Helpers for the GPU parity tests (device transfer, BF16 decoding and the
per-element tolerance).

GEMM acceptance, per output element, against the oracle's FP64 result:
    |c - ref| <= 2^-7 |ref| + 1e-3 rms(ref)
rms is taken over the whole output (real rows only for the grouped GEMM).
The 2^-7 term covers the BF16 write-back (at most 2^-9 relative) with margin
for FP32 accumulation-order effects across K/128 promoted block sums; the
rms term absorbs cancellation in elements whose exact value is near zero.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bf16_to_f64(t) -> np.ndarray:
    return t.view(torch.bfloat16).float().cpu().numpy().astype(np.float64)


def tolerance(c, ref, rows_mask=None):
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rows_mask is not None:
        c, ref = c[rows_mask], ref[rows_mask]
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return rms


def assert_close(c, ref, rms=None, what=""):
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(c - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 1e-3 * rms
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d/%d elements out of tolerance; first %s: got %s want %s"
                             % (what, int(bad.sum()), bad.size, idx.tolist(),
                                [c[tuple(i)] for i in idx], [ref[tuple(i)] for i in idx]))
    return float(np.max(err / (np.abs(ref) + rms))) if ref.size else 0.0


def tile_points(M, N, tile_m, tile_n, rng, rows=None):
    """One random point inside every tile_m x tile_n block of an M x N
    output (restricted to the given candidate rows when `rows` is set)."""
    pm, pn = [], []
    for m0 in range(0, M, tile_m):
        if rows is not None:
            cand = rows[(rows >= m0) & (rows < m0 + tile_m)]
            if cand.size == 0:
                continue
        n0 = np.arange(0, N, tile_n)
        if rows is not None:
            pm.append(rng.choice(cand, n0.size))
        else:
            pm.append(m0 + rng.integers(0, min(tile_m, M - m0), n0.size))
        pn.append(n0 + rng.integers(0, tile_n, n0.size) % np.minimum(tile_n, N - n0))
    return np.concatenate(pm).astype(np.int64), np.concatenate(pn).astype(np.int64)


def oracle_gemm_rows(orc, qa, sa, qb, sb, a_block_rows, threads=16):
    """orc.gemm_nt over slices of 128 rows of A handed to host threads (the
    oracle's C code releases the GIL): each output row is the oracle's own
    result for that row, only computed concurrently."""
    M = qa.shape[0]
    n_blk = (M + 127) // 128
    T = max(1, min(threads, os.cpu_count() or 1, n_blk))
    cuts = [128 * (n_blk * t // T) for t in range(T)] + [M]
    br = a_block_rows

    def part(t):
        r0, r1 = cuts[t], cuts[t + 1]
        return orc.gemm_nt(np.ascontiguousarray(qa[r0:r1]),
                           np.ascontiguousarray(sa[:, r0 // br:(r1 + br - 1) // br]),
                           qb, sb, a_block_rows=br)
    with cf.ThreadPoolExecutor(max_workers=T) as ex:
        return np.concatenate(list(ex.map(part, range(T))), axis=0)
