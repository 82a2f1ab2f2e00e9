"""Exact integer GEMM of quantized codes.

[P1] "Measurements": the INT4 path multiplies 4-bit activation codes with
4-bit weight codes on integer matrix units and rescales afterwards (rank-one
scale s_a * s_w for tensorwise formats). [P2] build table / file layout:
the W4A8 format multiplies 8-bit activation codes with asymmetric 4-bit
weights in groups of 16 along K. [P3] Quantization Method: SVDQuant W4A4
uses per-group scales, so the contraction splits into per-group partials.

Definitions:
  acc[m, n]     = sum_k qa[m, k] * qw[n, k]
  P[m, n, g]    = sum_{k in group g} qa[m, k] * (qw[n, k] - z[n, g])   (z = 0 if symmetric)

Computed exactly: float64 BLAS on integer-valued arrays is exact while every
partial sum stays below 2**53, which is asserted from the operand bounds.
"""
from __future__ import annotations

import numpy as np


def _assert_exact(qa: np.ndarray, qw: np.ndarray, K: int):
    bound = float(np.max(np.abs(qa), initial=0)) * float(np.max(np.abs(qw), initial=0)) * K
    if bound >= 2.0 ** 53:
        raise ValueError("integer GEMM bound exceeds exact float64 range")


def int_gemm(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc = qa @ qw.T, exact, int64. qa [M, K], qw [N, K] integer arrays."""
    qa = np.asarray(qa).astype(np.int64)
    qw = np.asarray(qw).astype(np.int64)
    if qa.shape[1] != qw.shape[1]:
        raise ValueError("K mismatch")
    _assert_exact(qa, qw, qa.shape[1])
    acc = qa.astype(np.float64) @ qw.astype(np.float64).T
    return np.rint(acc).astype(np.int64)


def group_partials(qa: np.ndarray, qw: np.ndarray, group: int,
                   zeros: np.ndarray | None = None) -> np.ndarray:
    """P[m, n, g] = sum_{k in g} qa[m, k] * (qw[n, k] - z[n, g]), exact int64.
    Memory is M*N*(K/group)*8 bytes: call it on row slices for large shapes."""
    qa = np.asarray(qa).astype(np.int64)
    qw = np.asarray(qw).astype(np.int64)
    M, K = qa.shape
    N = qw.shape[0]
    G = K // group
    w = qw.reshape(N, G, group)
    if zeros is not None:
        w = w - np.asarray(zeros).astype(np.int64)[:, :, None]
    a = qa.reshape(M, G, group)
    _assert_exact(a, w, group)
    out = np.empty((M, N, G), dtype=np.int64)
    for g in range(G):
        out[:, :, g] = np.rint(a[:, g, :].astype(np.float64) @ w[:, g, :].astype(np.float64).T)
    return out
