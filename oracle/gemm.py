"""W4A4 GEMM on INT4 codes: exact integer accumulation and the scale epilogue, float64.

Test infrastructure (see the package docstring): not part of the product path.

Sources (restated): "SpinQuant Guide: Learned Rotations for 4-Bit LLMs", section
"The Orthogonal Invariance Principle" (y = (W R^T)(R x), so a layer can run on the
rotated activation and the rotated weight) and "Production Engineering and Cluster
Deployment Best Practices" (weights rotated and packed to INT4 offline, the product
run as a low-bit GEMM); "SpinQuant: rotate before you round", section "Deployment
implications" (online: load packed low-bit weights, run the Hadamard transforms, run
the low-bit GEMM). With per-token activation scales sA and per-output-channel weight
scales sW, the dequantized product is
    out[m, n] = sA[m] * sW[n] * sum_k qA[m, k] * qW[n, k].

The integer sum is computed with a float64 matrix product: every partial sum is an
integer of magnitude at most K * 64, far below 2^53, so the result is exact.
"""

import numpy as np


def int_gemm(qa, qw):
    """acc[m, n] = sum_k qa[m, k] * qw[n, k], exact, returned as int64.

    qa: int codes [M, K]; qw: int codes [N, K] (both "K-contiguous", the NT layout).
    """
    qa = np.asarray(qa, dtype=np.float64)
    qw = np.asarray(qw, dtype=np.float64)
    if qa.ndim != 2 or qw.ndim != 2 or qa.shape[1] != qw.shape[1]:
        raise ValueError("qa must be [M, K] and qw [N, K]")
    k = qa.shape[1]
    bound = float(k) * max(np.max(np.abs(qa), initial=0.0), 1.0) * max(np.max(np.abs(qw), initial=0.0), 1.0)
    if bound >= 2.0 ** 53:
        raise ValueError("integer sums would not be exact in float64")
    return np.rint(qa @ qw.T).astype(np.int64)


def w4a4_gemm(qa, sa, qw, sw):
    """Dequantized W4A4 product.

    qa [M, K], qw [N, K]: int codes; sa [M], sw [N]: stored scales (any float dtype,
    upcast exactly). Returns (acc int64 [M, N], out float64 [M, N]).
    """
    acc = int_gemm(qa, qw)
    sa = np.asarray(sa, dtype=np.float64)
    sw = np.asarray(sw, dtype=np.float64)
    out = acc.astype(np.float64) * sa[:, None] * sw[None, :]
    return acc, out


def w4a8_gemm(qa, sa, qw, sw):
    """Dequantized W4A8 product: INT8 activation codes qa [M, K] (scale max/127 per
    token), INT4 weight codes qw [N, K]; the same exact integer sum and epilogue as
    ``w4a4_gemm`` (|sum| <= K * 128 * 8, exact in float64)."""
    return w4a4_gemm(qa, sa, qw, sw)



def w4a8_gemm_grouped(qa, sa, qw, sw_groups, group):
    """W4A8 product with group-wise weight scales ("SpinQuant, when rotations are worth
    learning": its ExecuTorch export quantizes weights to 4 bits in groups of 256 or 32
    input channels, with 8-bit dynamic activations):
        out[m, n] = sa[m] * sum_g sw_groups[n, g] * sum_{k in group g} qa[m, k] * qw[n, k]
    with group g covering k in [g * group, (g + 1) * group).

    qa int codes [M, K], qw int codes [N, K], sa [M], sw_groups [N, K / group].
    Returns (partial int64 [K / group, M, N], out float64 [M, N]); every partial sum is
    exact (float64 products of integers), the group sums are combined in float64.
    """
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    k = qa.shape[1]
    if group < 1 or k % group:
        raise ValueError("the group size must divide K")
    ng = k // group
    sa = np.asarray(sa, dtype=np.float64)
    sw = np.asarray(sw_groups, dtype=np.float64)
    if sw.shape != (qw.shape[0], ng):
        raise ValueError("sw_groups must be [N, K / group]")
    partial = np.stack([int_gemm(qa[:, g * group:(g + 1) * group], qw[:, g * group:(g + 1) * group])
                        for g in range(ng)])
    out = np.zeros(partial.shape[1:], dtype=np.float64)
    for g in range(ng):
        out += partial[g].astype(np.float64) * sw[None, :, g]
    return partial, out * sa[:, None]
