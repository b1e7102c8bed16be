"""Independent brute-force references used to pin the oracle on tiny inputs.

TEST INFRASTRUCTURE ONLY.  These deliberately take a different route from
``zp_oracle.c``: dense masked matrices and library routines (SciPy softmax,
scikit-learn cosine similarity, PyTorch scaled-dot-product attention in
double), and exhaustive search instead of sorting.  They are only meant for
small inputs.
"""
from __future__ import annotations

import itertools
from fractions import Fraction
from typing import Sequence

import numpy as np


def logical_rows(pool: np.ndarray, table: np.ndarray, head: int, length: int) -> np.ndarray:
    """Rows 0..length-1 of one request/head read through a block table, as float64."""
    nb, H, b, d = pool.shape
    if pool.dtype == np.uint16:
        vals = (pool.astype(np.uint32) << 16).view(np.float32)
    else:
        vals = pool
    j = np.arange(length)
    return vals[table[j // b], head, j % b].astype(np.float64)


def importance_dense(K: np.ndarray, Qw: np.ndarray) -> np.ndarray:
    """Observation-window importance from the dense masked attention matrix.

    K: [T][d] logical keys of one head.  Qw: [w][G][d] window queries of the
    head's group.  Builds the full (G*w) x T logit matrix with -inf above the
    causal diagonal (window row i sees slots <= T-w+i), applies SciPy's
    softmax per row, and averages the rows.
    """
    from scipy.special import softmax
    T, d = K.shape
    w, G, _ = Qw.shape
    rows = Qw.transpose(1, 0, 2).reshape(G * w, d)          # (g, i) row order
    X = rows @ K.T / np.sqrt(d)
    limit = np.tile(T - w + np.arange(w), G)                # p_i per row
    X = np.where(np.arange(T)[None, :] <= limit[:, None], X, -np.inf)
    return softmax(X, axis=1).mean(axis=0)


def lrs_sklearn(K: np.ndarray, b: int) -> np.ndarray:
    """In-block redundancy via scikit-learn's cosine_similarity (zero rows -> 0)."""
    from sklearn.metrics.pairwise import cosine_similarity
    T = K.shape[0]
    out = np.zeros(T)
    for n in range(T // b):
        blk = K[n * b:(n + 1) * b]
        S = cosine_similarity(blk)
        np.fill_diagonal(S, 0.0)
        out[n * b:(n + 1) * b] = S.sum(axis=1) / (b - 1)
    return out


def select_exhaustive(s: Sequence, k_sel: int) -> list:
    """Best k_sel-subset by exhaustive search: maximise (sum of s, -sum of slots).

    Exact for Fraction or integer scores.  Equivalent to "keep the largest
    scores, lower slot wins a tie" without ever sorting.
    """
    C = len(s)
    best, best_key = None, None
    for subset in itertools.combinations(range(C), k_sel):
        key = (sum(Fraction(s[j]) for j in subset), -sum(subset))
        if best_key is None or key > best_key:
            best, best_key = subset, key
    return sorted(best)


def decode_sdpa(K: np.ndarray, V: np.ndarray, q: np.ndarray, scale: float) -> np.ndarray:
    """Decode attention of one query head via PyTorch SDPA in double on the CPU."""
    import torch
    Kt = torch.from_numpy(np.ascontiguousarray(K))[None, None]
    Vt = torch.from_numpy(np.ascontiguousarray(V))[None, None]
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return o[0, 0, 0].numpy()
