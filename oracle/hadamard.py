"""Sylvester-Hadamard matrices and the explicit rotation y = H_n x / sqrt(n), in float64.

Test infrastructure (see the package docstring): not part of the product path.

Source: "Rotations: QuaRot, SpinQuant and incoherence", section "Hadamard matrices":
H_1 = [1]; H_2n is the 2x2 block matrix [[H_n, H_n], [H_n, -H_n]]; H_n / sqrt(n) is
orthogonal. The same page ("Why it's free: computational invariance") and "SpinQuant,
when rotations are worth learning" (section "Four rotation sites", R3 and R4) place the
fixed Hadamard online on Q/K after RoPE and on the down-projection input; only powers
of two are supported (the page's own note that the K-cache path asserts a power-of-two
head dimension), which is what this module accepts.

The rotation is a plain matrix product with the explicitly constructed matrix. For
large n the matrix is produced one block of columns at a time (to bound memory); every
output column is still the dot product of a row of x with the corresponding column of
H_n, so this is the definition, not a fast transform.
"""

import math

import numpy as np


def _check_pow2(n):
    if not isinstance(n, (int, np.integer)) or n < 1 or (n & (n - 1)) != 0:
        raise ValueError(f"Hadamard size must be a power of two >= 1, got {n!r}")


def sylvester(n):
    """H_n by the Sylvester recursion, entries +-1 as float64 (n a power of two)."""
    _check_pow2(n)
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_popcount(n):
    """Closed form of the Sylvester matrix: H[i, j] = (-1)^popcount(i AND j).

    Follows from the recursion by induction on the top bit of i and j (the -H_n block
    is exactly where both top bits are set). Used only as an independent cross-check
    of ``sylvester``.
    """
    _check_pow2(n)
    i = np.arange(n, dtype=np.int64)
    a = i[:, None] & i[None, :]
    parity = np.zeros_like(a)
    while np.any(a):
        parity ^= a & 1
        a >>= 1
    return 1.0 - 2.0 * parity.astype(np.float64)


def hadamard_column_block(n, col0, width):
    """Columns [col0, col0 + width) of H_n, built from the Sylvester recursion.

    H_n = H_{n/width} (x) H_width (Kronecker product, which is what unrolling the
    recursion gives), so column col0 + j of H_n is the Kronecker product of column
    col0 / width of H_{n/width} with column j of H_width.
    """
    _check_pow2(n)
    _check_pow2(width)
    if width > n or col0 % width != 0:
        raise ValueError("column block must be aligned and inside the matrix")
    outer = sylvester(n // width)[:, col0 // width]
    return np.kron(outer[:, None], sylvester(width))


def rotate(x, normalize=True, block=4096):
    """Rotate every row of x by the Sylvester Hadamard: y = x H_n (/ sqrt(n)).

    x: array [..., n] (any real dtype; upcast to float64 exactly).
    Because H_n is symmetric, x H_n (row form) equals (H_n x^T)^T (column form).
    normalize: divide by sqrt(n) so the map is orthogonal.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    _check_pow2(n)
    rows = x.reshape(-1, n)
    if n <= block:
        y = rows @ sylvester(n)
    else:
        y = np.empty_like(rows)
        for c in range(0, n, block):
            y[:, c:c + block] = rows @ hadamard_column_block(n, c, block)
    if normalize:
        y = y / math.sqrt(n)
    return y.reshape(x.shape)


def rotate_signed(x, signs):
    """Randomized Hadamard rotation of every row: y = H_n diag(signs) x / sqrt(n).

    "Rotations: QuaRot, SpinQuant and incoherence", section "Hadamard matrices": flipping
    the signs of the coordinates by a random +-1 diagonal before the normalised Hadamard
    makes the largest output entry close to the row's RMS with high probability, also for
    inputs that the plain transform would leave coherent. signs: [n] of +-1.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    if s.shape != (x.shape[-1],) or not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be a vector of +-1 of the row length")
    return rotate(x * s)

