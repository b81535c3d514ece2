"""Rotary position embedding ahead of the R3 rotation, computed from its definition.

Test infrastructure (see the package docstring): not part of the product path.

"SpinQuant, when rotations are worth learning", section "Four rotation sites": R3 is a
fixed Hadamard applied to queries and keys after RoPE. "SpinQuant Guide: Learned
Rotations for 4-Bit LLMs" (section on RoPE compatibility with 4-bit KV caching): RoPE
rotates 2-D coordinate pairs by position-dependent angles. The pages do not fix which
coordinates pair up; this operation pairs element i with element i + D/2 (i < D/2), the
half-split layout, and takes the angles as caller-supplied tables cos[p, i], sin[p, i]
(p = position, i < D/2):

    x'[i]       = x[i] cos - x[i + D/2] sin
    x'[i + D/2] = x[i + D/2] cos + x[i] sin

The rotated pair is then stored in the input's 16-bit format (what the R3 rotation reads
when RoPE runs as its own step). ``rope_16bit`` is that definition: the map evaluated
exactly (float64 products of 16-bit inputs and float32 table entries, one float64 sum),
rounded once to the format, nearest even.

A device evaluates the map in float32 before the rounding. Its result can then fall on
the other side of a rounding midpoint of the format, but only where the exact value lies
within the float32 evaluation error of that midpoint; ``rope_16bit_ambiguous`` marks
those elements and gives the other neighbour, so a comparison can accept either there
and demand equality everywhere else.
"""

import numpy as np

# significand bits (with the leading one) and the frexp exponent of the smallest normal
_FORMATS = {"bfloat16": (8, -125), "float16": (11, -13)}


def rope_exact(x, cos, sin):
    """float64 half-split RoPE of x [..., D] with cos/sin [..., D/2] (broadcast)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a, b = x[..., : d // 2], x[..., d // 2:]
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _grid(v, fmt):
    """The two values of the format's grid around v (lo <= v < hi, lo on the grid) and
    the spacing, float64. Finite values in the format's normal or subnormal range."""
    p, emin = _FORMATS[fmt]
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    e = np.maximum(e, emin)
    spacing = np.ldexp(np.ones_like(v), e - p)
    lo = np.floor(v / spacing) * spacing
    return lo, lo + spacing, spacing


def round_to_format(v, fmt):
    """float64 values rounded to nearest 'bfloat16' or 'float16' value, ties to the even
    significand, returned as float64 (no overflow handling: finite, in-range values)."""
    v = np.asarray(v, dtype=np.float64)
    lo, hi, spacing = _grid(v, fmt)
    mid = lo + 0.5 * spacing
    lo_even = np.mod(np.rint(lo / spacing), 2.0) == 0.0
    up = (v > mid) | ((v == mid) & ~lo_even)
    out = np.where(up, hi, lo)
    return np.where(v == 0.0, v, out)


def rope_16bit(x, cos, sin, fmt):
    """RoPE of x [..., D] (values exact in ``fmt``) with float32 tables cos/sin [..., D/2],
    evaluated exactly and rounded once to ``fmt`` ('bfloat16' or 'float16'); float64."""
    return round_to_format(rope_exact(x, cos, sin), fmt)


def rope_16bit_ambiguous(x, cos, sin, fmt):
    """(value, other, mask): ``value`` is rope_16bit; ``mask`` marks the elements whose
    exact value lies within the error bound of a float32 evaluation (products and sum each
    rounded, or fused) of a rounding midpoint of ``fmt``, where such an evaluation may
    round to ``other``, the neighbour on the far side of that midpoint.

    The bound for fl(fl(a) +- fl(b)) is 2u (|a| + |b|)(1 + u), u = 2^-24, plus three
    float32 subnormal steps (2^-149) for products that underflow."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a, b = x[..., : d // 2], x[..., d // 2:]
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    exact = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    mag = np.concatenate([np.abs(a * c) + np.abs(b * s), np.abs(b * c) + np.abs(a * s)], axis=-1)
    bound = 2.0 ** -23 * mag * (1.0 + 2.0 ** -23) + 3.0 * 2.0 ** -149
    value = round_to_format(exact, fmt)
    lo, hi, spacing = _grid(exact, fmt)
    mid = lo + 0.5 * spacing
    mask = np.abs(exact - mid) <= bound
    other = np.where(value == lo, hi, lo)
    return value, np.where(mask, other, value), mask
