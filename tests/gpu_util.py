"""Helpers for the GPU parity tests (device transfer, BF16 decoding and the
per-element tolerance).

GEMM acceptance, per output element, against the oracle's FP64 result:
    |c - ref| <= 2^-7 |ref| + 1e-3 rms(ref)
rms is taken over the whole output (real rows only for the grouped GEMM).
The 2^-7 term covers the BF16 write-back (at most 2^-9 relative) with margin
for FP32 accumulation-order effects across K/128 promoted block sums; the
rms term absorbs cancellation in elements whose exact value is near zero.
"""
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
