"""ConvRot rotation: a block-diagonal regular Hadamard transform along K.

[P1] intro: weights and activations are both rotated with the same
regular Hadamard matrix applied to contiguous groups of 256 input channels;
activations are rotated online, weights once offline. [P5] Format and [P2]
group-size notes: the group size is 256 (W4A4 also accepts 16, 64 and 1024).

The pages name the matrix only as "regular Hadamard" and give neither its
entries nor an evaluation order. Readings taken here:

* Matrix. For n = 4**d, H = (-1)**d * D @ S @ D, where S is the Sylvester
  Hadamard matrix S[i, j] = (-1)**popcount(i & j) and D is diagonal with
  D[j] = (-1)**z(j), z(j) = the number of zero digits among the d base-4
  digits of j. H is symmetric, has +-1 entries, H @ H.T = n*I and every row
  and column sums to +sqrt(n): it is a regular Hadamard matrix, and the sizes
  the pages allow (16, 64, 256, 1024) are exactly the powers of four, the
  square orders a regular Hadamard matrix needs.
* Normalisation. The orthonormal rotation is H / sqrt(n). `rotate` returns
  the unnormalised H @ x; the power-of-two 1/sqrt(n) is carried by the stored
  quantization scale (see quant.py), which leaves every code unchanged.
* Evaluation order (fixes float32 rounding, so the codes are reproducible):
  x <- D*x; then the in-place butterfly (x_i, x_{i+h}) <- (x_i + x_{i+h},
  x_i - x_{i+h}) for h = 1, 2, 4, ..., n/2 in that order, each sum rounded to
  float32; then x <- D*x and the overall sign (-1)**d. Sign flips are exact.
"""
from __future__ import annotations

import numpy as np

ALLOWED_GROUPS = (16, 64, 256, 1024)


def n_digits(n: int) -> int:
    """Number of base-4 digits d with n == 4**d (n must be a power of four)."""
    d = 0
    m = 1
    while m < n:
        m *= 4
        d += 1
    if m != n:
        raise ValueError(f"group size {n} is not a power of four")
    return d


def digit_signs(n: int) -> np.ndarray:
    """D[j] = (-1)**(number of zero base-4 digits of j), j in [0, n)."""
    d = n_digits(n)
    out = np.empty(n, dtype=np.int64)
    for j in range(n):
        zeros = 0
        t = j
        for _ in range(d):
            if t % 4 == 0:
                zeros += 1
            t //= 4
        out[j] = -1 if zeros % 2 else 1
    return out


def sylvester(n: int) -> np.ndarray:
    """S[i, j] = (-1)**popcount(i & j)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    a = i & j
    pc = np.zeros_like(a)
    while np.any(a):
        pc += a & 1
        a = a >> 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def regular_hadamard(n: int) -> np.ndarray:
    """The explicit n x n regular Hadamard matrix H (int64 entries +-1)."""
    d = n_digits(n)
    dv = digit_signs(n)
    sign = -1 if d % 2 else 1
    return sign * (dv[:, None] * sylvester(n) * dv[None, :])


def rotate(x: np.ndarray, group: int = 256) -> np.ndarray:
    """Unnormalised group-wise rotation y[r, g*n:(g+1)*n] = H @ x[r, g*n:(g+1)*n],
    evaluated in float32 in the fixed butterfly order stated in the module
    docstring. x: float32 [rows, K] with K % group == 0. Returns float32."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % group != 0:
        raise ValueError("rotate expects [rows, K] with K a multiple of the group size")
    rows, K = x.shape
    d = n_digits(group)
    dv = digit_signs(group).astype(np.float32)
    y = x.reshape(rows, K // group, group) * dv          # exact sign flips
    h = 1
    while h < group:
        blocks = y.reshape(rows, K // group, group // (2 * h), 2, h)
        lo = blocks[:, :, :, 0, :]                          # elements i   (bit h clear)
        hi = blocks[:, :, :, 1, :]                          # elements i+h (bit h set)
        y = np.stack([lo + hi, lo - hi], axis=3)            # float32 adds, RNE
        h *= 2
    y = y.reshape(rows, K // group, group) * dv
    if d % 2:
        y = -y
    return np.ascontiguousarray(y.reshape(rows, K), dtype=np.float32)
