"""Rotary position embedding ahead of the R3 rotation, as the fused operation defines it.

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

The fused kernel evaluates this in float32 -- each product rounded, then the sum rounded,
no fused multiply-add -- and rounds x' to the input's 16-bit format (nearest even) before
the Hadamard, i.e. exactly what an unfused RoPE kernel writing bf16/fp16 would hand to
kv_rotate_quant. ``rope_16bit`` reproduces that arithmetic step by step with NumPy float32
operations (IEEE binary32, the same rounding), so its output is the exact expected input
of the rotation; ``rope_exact`` is the same map in float64 for the pins.
"""

import numpy as np


def rope_exact(x, cos, sin):
    """float64 half-split RoPE of x [..., D] with cos/sin [..., D/2] (broadcast)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a, b = x[..., : d // 2], x[..., d // 2:]
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _round_f32_to_16bit(v, fmt):
    """Nearest-even rounding of float32 values to bfloat16 or float16, returned as float64."""
    v = np.asarray(v, dtype=np.float32)
    if fmt == "float16":
        return v.astype(np.float16).astype(np.float64)
    bits = v.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def rope_16bit(x, cos, sin, fmt):
    """The fused kernel's RoPE: float32 arithmetic (rounded products, rounded sum), result
    rounded to the 16-bit input format ``fmt`` ('bfloat16' or 'float16'), as float64.

    x [..., D] holds values exactly representable in ``fmt``; cos/sin [..., D/2] float32."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    a, b = x[..., : d // 2], x[..., d // 2:]
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    lo = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    hi = (b * c).astype(np.float32) + (a * s).astype(np.float32)
    return _round_f32_to_16bit(np.concatenate([lo, hi], axis=-1).astype(np.float32), fmt)
