"""Hadamard rotations of rows whose length is not a power of two, in float64.

Test infrastructure (see the package docstring): not part of the product path.

Source: "Rotations: QuaRot, SpinQuant and incoherence", section "Hadamard matrices":
lengths that are not powers of two are rotated by the Kronecker product of a
power-of-two Hadamard matrix with a small known Hadamard matrix. The page names neither
the small matrix nor the order of the factors; the readings fixed here are:

* n = m * p with p a power of two; the rotation is y = (H_m (x) H_p) x / sqrt(n), where
  element a * p + b of a row is index (a, b) of the product (a in [0, m), b in [0, p)),
  H_p is the Sylvester matrix and H_m is a Paley matrix.
* m is the smallest of 4 o, 8 o, 16 o, ... (o the odd part of n, m <= 256, m dividing n)
  for which a construction below exists: Paley I when m - 1 is a prime q = 3 (mod 4),
  else Paley II when m / 2 - 1 is a prime q = 1 (mod 4), or the Goethals-Seidel matrix
  of order 172. A power of two has m = 1 (the Sylvester matrix alone).
* Paley I: H = I + [[0, j^T], [-j, Q]], with j the all-ones column and Q the Jacobsthal
  matrix Q[a][b] = chi(a - b), chi the quadratic character of GF(q).
* Paley II: C = [[0, j^T], [j, Q]] (symmetric for q = 1 mod 4); every 0 of C becomes the
  2 x 2 block [[1, -1], [-1, -1]] and every +-1 becomes +-[[1, 1], [1, -1]], block (R, C)
  of H covering rows 2R, 2R + 1 and columns 2C, 2C + 1.

The Paley matrices are the textbook constructions (R. E. A. C. Paley, "On orthogonal
matrices", 1933), written here from their definitions.

Order 172 = 4 * 43 has no Paley construction over a prime field (171 and 85 are not
prime), yet 11008 = 172 * 64 is a common FFN width, so the rule also takes the
Goethals-Seidel array (J. M. Goethals and J. J. Seidel, "Orthogonal matrices with zero
diagonal", 1967): four circulant +-1 matrices A, B, C, D of order 43 whose periodic
autocorrelations add up to zero at every nonzero shift (A A^T + B B^T + C C^T + D D^T =
172 I), placed as

    [[ A,    B R,    C R,    D R  ],
     [-B R,  A,      D^T R, -C^T R],
     [-C R, -D^T R,  A,      B^T R],
     [-D R,  C^T R, -B^T R,  A    ]]

with R the back-diagonal permutation. The four first rows are taken constant on the
cosets of the subgroup of order 7 of the multiplicative group mod 43 (a cyclotomic
choice that makes the search small): ``gs_first_rows`` fixes them as the
lexicographically first quadruple satisfying the condition, by exhaustive search.
"""

import math

import numpy as np

from .hadamard import sylvester


def is_prime(v):
    """Trial division."""
    if v < 2:
        return False
    d = 2
    while d * d <= v:
        if v % d == 0:
            return False
        d += 1
    return True


def legendre(a, q):
    """Quadratic character chi(a) of GF(q), q an odd prime, by Euler's criterion:
    a^((q-1)/2) mod q is 1 for a nonzero square, q - 1 for a non-square, 0 for a = 0."""
    r = pow(int(a) % q, (q - 1) // 2, q)
    return 0 if r == 0 else (1 if r == 1 else -1)


def paley_kind(m):
    """(q, 1) for Paley I, (q, 2) for Paley II, or None when neither applies to order m."""
    if m >= 4 and is_prime(m - 1) and (m - 1) % 4 == 3:
        return m - 1, 1
    if m >= 4 and m % 2 == 0 and is_prime(m // 2 - 1) and (m // 2 - 1) % 4 == 1:
        return m // 2 - 1, 2
    return None


GS_ORDER = 172   # 4 * 43: the Goethals-Seidel factor
GS_P = 43        # order of its circulant blocks
GS_H = 7         # order of the subgroup whose cosets the first rows are constant on


def primitive_root(p):
    """Smallest generator of the multiplicative group mod the prime p."""
    for g in range(2, p):
        if len({pow(g, k, p) for k in range(1, p)}) == p - 1:
            return g
    raise ValueError(p)


def gs_coset_sequence(code, p=GS_P, h=GS_H):
    """The +-1 sequence of length p for a code: bit 0 gives the entry at 0, bit j (j >= 1)
    the entries on the j-th coset of the subgroup of order h of (Z/p)^*, cosets ordered by
    their smallest element; a set bit is +1."""
    g = primitive_root(p)
    sub = {pow(g, (p - 1) // h * k, p) for k in range(h)}
    x = np.empty(p, dtype=np.int64)
    x[0] = 1 if code & 1 else -1
    seen, j = set(), 0
    for t in range(1, p):
        if t in seen:
            continue
        j += 1
        coset = {(t * u) % p for u in sub}
        seen |= coset
        x[sorted(coset)] = 1 if (code >> j) & 1 else -1
    return x


def periodic_autocorrelation(x):
    """PAF(s) = sum_t x[t] x[(t + s) mod p] for s = 1 .. p - 1."""
    x = np.asarray(x, dtype=np.int64)
    return np.array([int(np.dot(x, np.roll(x, -s))) for s in range(1, len(x))], dtype=np.int64)


_GS_ROWS = None


def gs_first_rows():
    """The four first rows (A, B, C, D) of the order-172 factor: over codes i <= j <= k <= l
    of ``gs_coset_sequence`` in lexicographic order, the first quadruple whose periodic
    autocorrelations add up to zero at every nonzero shift. int64 array [4, 43]."""
    global _GS_ROWS
    if _GS_ROWS is None:
        ncodes = 1 << (1 + (GS_P - 1) // GS_H)
        seqs = [gs_coset_sequence(v) for v in range(ncodes)]
        paf = np.array([periodic_autocorrelation(x) for x in seqs])
        by_key = {}
        for l in range(ncodes):
            by_key.setdefault(paf[l].tobytes(), []).append(l)
        found = None
        for i in range(ncodes):
            for j in range(i, ncodes):
                for k in range(j, ncodes):
                    need = -(paf[i] + paf[j] + paf[k])
                    ls = [l for l in by_key.get(need.tobytes(), []) if l >= k]
                    if ls:
                        found = (i, j, k, ls[0])
                        break
                if found:
                    break
            if found:
                break
        if found is None:
            raise RuntimeError("no quadruple")
        _GS_ROWS = np.array([seqs[c] for c in found])
    return _GS_ROWS.copy()


def circulant(x):
    """X[i][j] = x[(j - i) mod n]."""
    n = len(x)
    return np.array([[x[(j - i) % n] for j in range(n)] for i in range(n)], dtype=np.float64)


def goethals_seidel_hadamard(rows=None):
    """The Goethals-Seidel array above on the circulants of ``rows`` (default
    ``gs_first_rows()``); float64 [4n, 4n]."""
    a, b, c, d = [circulant(x) for x in (gs_first_rows() if rows is None else rows)]
    n = a.shape[0]
    r = np.fliplr(np.eye(n))
    return np.block([[a, b @ r, c @ r, d @ r],
                     [-b @ r, a, d.T @ r, -c.T @ r],
                     [-c @ r, -d.T @ r, a, b.T @ r],
                     [-d @ r, c.T @ r, -b.T @ r, a]])


def jacobsthal(q):
    """Q[a][b] = chi(a - b), a, b in GF(q)."""
    chi = [legendre(d, q) for d in range(q)]
    return np.array([[chi[(a - b) % q] for b in range(q)] for a in range(q)], dtype=np.float64)


def paley_hadamard(m):
    """The Paley Hadamard matrix of order m (entries +-1, float64)."""
    kind = paley_kind(m)
    if kind is None:
        raise ValueError(f"no Paley construction of order {m}")
    q, k = kind
    Q = jacobsthal(q)
    if k == 1:
        S = np.zeros((m, m))
        S[0, 1:] = 1.0
        S[1:, 0] = -1.0
        S[1:, 1:] = Q
        return np.eye(m) + S
    C = np.zeros((q + 1, q + 1))
    C[0, 1:] = 1.0
    C[1:, 0] = 1.0
    C[1:, 1:] = Q
    zero_block = np.array([[1.0, -1.0], [-1.0, -1.0]])
    one_block = np.array([[1.0, 1.0], [1.0, -1.0]])
    H = np.empty((m, m))
    for R in range(q + 1):
        for Cc in range(q + 1):
            v = C[R, Cc]
            H[2 * R:2 * R + 2, 2 * Cc:2 * Cc + 2] = zero_block if v == 0 else v * one_block
    return H


def kron_factor(n):
    """m for a row length n (1 for a power of two), or None when the rule finds none."""
    if n < 1:
        return None
    if n & (n - 1) == 0:
        return 1
    o = n
    while o % 2 == 0:
        o //= 2
    m = 4 * o
    while m <= 256 and n % m == 0:
        if has_construction(m):
            return m
        m *= 2
    return None


def has_construction(m):
    """Orders the rule can use: Paley I or II over a prime field, or the Goethals-Seidel
    order 172."""
    return m == GS_ORDER or paley_kind(m) is not None


def small_hadamard(m):
    """H_m of the rule: the Goethals-Seidel matrix for 172, else the Paley matrix."""
    return goethals_seidel_hadamard() if m == GS_ORDER else paley_hadamard(m)


def kron_hadamard(n):
    """The full n x n matrix H_m (x) H_p (explicit; small n only)."""
    m = kron_factor(n)
    if m is None:
        raise ValueError(f"no supported factorization of {n}")
    hm = np.ones((1, 1)) if m == 1 else small_hadamard(m)
    return np.kron(hm, sylvester(n // m))


def rotate_kron(x):
    """y = (H_m (x) H_p) x / sqrt(n) for every row of x [..., n], by the mixed-product
    property: H_p applied to each of the m blocks of p elements, then H_m across the
    blocks (two matrix products, no fast transform)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    m = kron_factor(n)
    if m is None:
        raise ValueError(f"no supported factorization of {n}")
    p = n // m
    hm = np.ones((1, 1)) if m == 1 else small_hadamard(m)
    blocks = x.reshape(-1, m, p) @ sylvester(p)          # H_p is symmetric
    y = np.einsum("ac,rcb->rab", hm, blocks)              # (H_m Y)[a, b] = sum_c H_m[a, c] Y[c, b]
    return (y / math.sqrt(n)).reshape(x.shape)
