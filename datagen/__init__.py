"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This module draws random numbers only; it contains none of the method's
arithmetic (no scaling, rounding, encoding or products), so the oracle and the
GPU path may both consume its arrays without sharing any computation.

Recipes (all float32 on the host, numpy PCG64 streams keyed by (seed, stream)):

* dense operands: i.i.d. normal with a given standard deviation (activations
  sigma=1, weights sigma=0.02), the shapes of LLM projection layers;
* outlier activations: Student-t with 3 degrees of freedom, with 1% of the K
  channels (round(0.01*K), chosen without replacement) multiplied by 100;
* MoE routing: each token picks ``topk`` distinct experts uniformly at random;
  rows are ordered by (expert, token) and every expert's group is padded with
  zero rows up to a multiple of the alignment (128), padding rows carrying
  expert id -1.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def normal(shape, sigma: float = 1.0, seed: int = 0, stream: int = 0) -> np.ndarray:
    """i.i.d. N(0, sigma^2), float32, C-contiguous."""
    x = rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return np.ascontiguousarray(x)


def student_t_outliers(rows: int, cols: int, nu: float = 3.0, frac: float = 0.01,
                       factor: float = 100.0, seed: int = 0, stream: int = 0):
    """Heavy-tailed activations with a few hot K channels.
    Returns (x float32 [rows, cols], hot channel indices)."""
    g = rng(seed, stream)
    x = g.standard_t(nu, size=(rows, cols)).astype(np.float32)
    n_hot = int(round(frac * cols))
    hot = np.sort(g.choice(cols, size=n_hot, replace=False))
    x[:, hot] *= np.float32(factor)
    return np.ascontiguousarray(x), hot


def moe_routing(num_tokens: int, num_experts: int, topk: int, align: int = 128,
                seed: int = 0, stream: int = 0):
    """Uniform top-k routing, grouped contiguously along M.

    Returns a dict with
      m_indices  int32 [M_total]: expert id per row, -1 for padding rows
      row_token  int64 [M_total]: source token per row, -1 for padding rows
      counts     int64 [E]: routed rows per expert (before padding)
      padded     int64 [E]: rows per expert after padding to ``align``
    """
    g = rng(seed, stream)
    keys = g.random((num_tokens, num_experts))
    choice = np.argsort(keys, axis=1)[:, :topk]          # distinct experts per token
    tok = np.repeat(np.arange(num_tokens), topk)
    exp = choice.reshape(-1)
    order = np.lexsort((tok, exp))                        # by expert, then token
    tok, exp = tok[order], exp[order]
    counts = np.bincount(exp, minlength=num_experts).astype(np.int64)
    padded = ((counts + align - 1) // align) * align
    m_total = int(padded.sum())
    m_indices = np.full(m_total, -1, dtype=np.int32)
    row_token = np.full(m_total, -1, dtype=np.int64)
    start = 0
    pos = 0
    for e in range(num_experts):
        c = int(counts[e])
        m_indices[start:start + c] = e
        row_token[start:start + c] = tok[pos:pos + c]
        pos += c
        start += int(padded[e])
    return {"m_indices": m_indices, "row_token": row_token,
            "counts": counts, "padded": padded}


def gather_rows(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """Rows of x picked by row_token; rows with token -1 are zero."""
    out = np.zeros((row_token.shape[0], x.shape[1]), dtype=x.dtype)
    real = row_token >= 0
    out[real] = x[row_token[real]]
    return out
