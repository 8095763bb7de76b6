"""Dense fp64 softmax attention: the plain definition, no paging, no tiling.

For each query row i and head h over a token set V:

    out[i, h, :] = sum_j exp(s_j - m) v[j, h, :] / sum_j exp(s_j - m),
    s_j = q[i, h, :] . k[j, h, :] / sqrt(D),   m = max_j s_j.

The paged kernel on the pages reads only the listed pages and never builds a
dense K/V ([P2] "FlashInfer Kernel Execution"; [P1] "FlashInfer Paged-Kernel
Integration"), and the force_fp32 path gathers the pages into dense tensors and
runs plain attention for numerical validation ([P2] "Memory Efficiency
Analysis").  That plain attention, over the rule-derived visible set, is what
this module computes.  The 1/sqrt(D) scale is the standard scaled dot-product
softmax; the pages do not print a different one.

Query rows are processed in chunks so that the score matrix of a long key set
is never held whole; chunking does not change any value (each row is computed
independently).
"""
from __future__ import annotations

import math

import numpy as np


def dense_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         scale: float | None = None) -> np.ndarray:
    """Single head.  q [Nq, D], k [Nk, D], v [Nk, Dv] -> [Nq, Dv], all fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        raise ValueError("empty key set: softmax undefined")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    s = (q @ k.T) * scale                      # [Nq, Nk]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e @ v) / e.sum(axis=1, keepdims=True)


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    scale: float | None = None, row_chunk: int = 256) -> np.ndarray:
    """Multi-head.  q [Nq, H, D], k [Nk, H, D], v [Nk, H, D] -> [Nq, H, D] fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, H, D = q.shape
    out = np.empty((nq, H, v.shape[2]), dtype=np.float64)
    for h in range(H):
        kh = np.ascontiguousarray(k[:, h, :])
        vh = np.ascontiguousarray(v[:, h, :])
        for r0 in range(0, nq, row_chunk):
            r1 = min(nq, r0 + row_chunk)
            out[r0:r1, h, :] = dense_attention_rows(q[r0:r1, h, :], kh, vh, scale)
    return out
