"""Pins of oracle.hadamard against mathematics the pages fix.

The pages ([P1] intro; [P5] Format; [P2] group-size note) fix: a *regular*
Hadamard matrix, applied to contiguous groups of 256 channels (W4A4 also
16/64/1024), the same on weights and activations. A regular Hadamard matrix
has +-1 entries, H H^T = n I and constant row and column sums (sqrt(n)).
"""
import numpy as np
import pytest

from oracle import hadamard


@pytest.mark.parametrize("n", [16, 64, 256, 1024])
def test_regular_hadamard_identities(n):
    H = hadamard.regular_hadamard(n)
    assert H.shape == (n, n)
    assert set(np.unique(H)) == {-1, 1}
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64))
    r = int(round(np.sqrt(n)))
    assert np.all(H.sum(axis=1) == r)
    assert np.all(H.sum(axis=0) == r)


def test_order_four_by_hand():
    # d = 1 digit. S4 rows: [1 1 1 1], [1 -1 1 -1], [1 1 -1 -1], [1 -1 -1 1];
    # D = diag(-1, 1, 1, 1) (only j = 0 has a zero digit); H = -D S D:
    # row 0: -(d0 d_j S[0,j]) = -(1, -1, -1, -1) = (-1, 1, 1, 1)
    # row 1: -(-1, -1, 1, -1) = (1, 1, -1, 1)
    # row 2: -(-1, 1, -1, -1) = (1, -1, 1, 1)
    # row 3: -(-1, -1, -1, 1) = (1, 1, 1, -1)
    expect = np.array([[-1, 1, 1, 1], [1, 1, -1, 1], [1, -1, 1, 1], [1, 1, 1, -1]])
    assert np.array_equal(hadamard.regular_hadamard(4), expect)


def test_order_sixteen_first_row_by_hand():
    # d = 2 digits (even, no overall sign). H16 = (D4 S4 D4) kron (D4 S4 D4);
    # row 0 of D4 S4 D4 is (1, -1, -1, -1), so row 0 of H16 is its Kronecker square.
    r = np.array([1, -1, -1, -1])
    assert np.array_equal(hadamard.regular_hadamard(16)[0], np.kron(r, r))


@pytest.mark.parametrize("n", [16, 64, 256, 1024])
def test_fwht_equals_matrix_on_basis_vectors(n):
    # Integer inputs are summed exactly, so the fast transform of e_j must be
    # column j of H bit for bit (a wrong sign vector, pairing or overall sign fails).
    H = hadamard.regular_hadamard(n)
    y = hadamard.rotate(np.eye(n, dtype=np.float32), n)   # row j = H e_j = column j
    assert np.array_equal(y, H.T.astype(np.float32))


def test_fwht_matches_fp64_matrix_product():
    g = np.random.default_rng(1)
    x = g.standard_normal((8, 1024)).astype(np.float32)
    x[:, 7] *= 30
    y = hadamard.rotate(x, 256).astype(np.float64)
    H = hadamard.regular_hadamard(256).astype(np.float64)
    ref = (x.astype(np.float64).reshape(8, 4, 256) @ H.T).reshape(8, 1024)
    err = np.abs(y - ref).max() / np.abs(ref).max()
    assert err < 1e-6


def test_joint_rotation_preserves_product():
    # The reason ConvRot is allowed at all: with R = H/16 orthogonal,
    # (X R^T)(W R^T)^T = X W^T. Checked in float64 with the explicit matrix.
    g = np.random.default_rng(2)
    X = g.standard_normal((5, 512))
    W = g.standard_normal((7, 512))
    R = hadamard.regular_hadamard(256).astype(np.float64) / 16.0
    Xr = (X.reshape(5, 2, 256) @ R.T).reshape(5, 512)
    Wr = (W.reshape(7, 2, 256) @ R.T).reshape(7, 512)
    assert np.allclose(Xr @ Wr.T, X @ W.T, rtol=1e-12, atol=1e-12)


def _recursive_fp32(x, dv, sign):
    """Independent brute-force statement of the same evaluation order:
    Sylvester recursion on halves, each half transformed first, the halves
    combined last, every sum rounded to float32 (np.float32 scalars)."""
    def syl(v):
        n = len(v)
        if n == 1:
            return [v[0]]
        a = syl(v[: n // 2])
        b = syl(v[n // 2:])
        return [np.float32(p + q) for p, q in zip(a, b)] + [np.float32(p - q) for p, q in zip(a, b)]
    v = [np.float32(d * t) for d, t in zip(dv, x)]
    out = syl(v)
    return np.array([np.float32(sign * d * t) for d, t in zip(dv, out)], dtype=np.float32)


def test_butterfly_order_bit_exact_vs_recursive_bruteforce():
    g = np.random.default_rng(3)
    x = (g.standard_normal((3, 256)) * np.exp(g.standard_normal((3, 256)) * 3)).astype(np.float32)
    dv = hadamard.digit_signs(256).astype(np.float32)
    y = hadamard.rotate(x, 256)
    for r in range(3):
        assert np.array_equal(y[r], _recursive_fp32(list(x[r]), list(dv), 1.0))


def test_butterfly_order_matters():
    # The pin above has teeth: running the stages in the reverse order rounds
    # differently on wide-dynamic-range float32 inputs.
    g = np.random.default_rng(4)
    x = (g.standard_normal((4, 256)) * np.exp(g.standard_normal((4, 256)) * 3)).astype(np.float32)
    dv = hadamard.digit_signs(256).astype(np.float32)
    y = (x * dv).reshape(4, 256)
    h = 128
    while h >= 1:
        b = y.reshape(4, 256 // (2 * h), 2, h)
        y = np.stack([b[:, :, 0] + b[:, :, 1], b[:, :, 0] - b[:, :, 1]], axis=2).reshape(4, 256)
        h //= 2
    rev = y * dv
    assert not np.array_equal(rev, hadamard.rotate(x, 256))
    assert np.allclose(rev, hadamard.rotate(x, 256), rtol=1e-5, atol=1e-3)


def test_rejects_non_power_of_four():
    with pytest.raises(ValueError):
        hadamard.regular_hadamard(128)
    with pytest.raises(ValueError):
        hadamard.rotate(np.zeros((1, 300), np.float32), 256)
