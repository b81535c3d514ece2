"""Per-row symmetric absmax INT4 quantization, nibble packing and the fused
rotate-then-quantize pipeline, in float64.

Test infrastructure (see the package docstring): not part of the product path.

Sources (all restated, none quoted):

* "SpinQuant Guide: Learned Rotations for 4-Bit LLMs", outlier-curse figure and the
  step-size equation: the INT4 grid is [-8, 7] and the step is max|X| / (2^(b-1) - 1),
  i.e. max|X| / 7 at b = 4 (the figure works 184.50 / 7 = 26.36).
* Same page, ``uniform_quantize_int4`` listing: the scale is floored at 1e-8, values
  are divided by the scale, clamped to [-8, 7] and rounded with ``torch.round``
  (round half to even), then multiplied back by the scale to dequantize.
* "Rotations: QuaRot, SpinQuant and incoherence", worked example "a hidden state with
  an outlier channel": the scale is per token (one per 4096-wide row), and the INT4
  step there is 60 / 7.
* Storage of the codes two per byte, low nibble first, two's complement, and scales in
  fp32 or fp16 (round to nearest even) is the format of the workloads this library
  serves; it is a reading, listed with the others in the design notes.

Readings fixed here where the pages are silent:

* Codes are computed against the scale *as stored* (rounded to its storage dtype), so
  dequantization q * s_stored lands on the grid the consumer GEMM uses.
* A stored scale of exactly 0 (fp16 underflow of a near-zero row) gives all-zero codes.
* Clamp-then-round (the listing's order) equals round-then-clamp for integer bounds;
  the tests check that property.
"""

import numpy as np

from .hadamard import rotate, rotate_signed
from .kron import rotate_kron

SCALE_FLOOR = 1e-8
QMIN = -8
QMAX = 7

_SCALE_DTYPES = {"float32": np.float32, "float16": np.float16}


def qrange(bits=4):
    """Symmetric signed grid of a b-bit code: [-2^(b-1), 2^(b-1) - 1] ("SpinQuant Guide:
    Learned Rotations for 4-Bit LLMs", step-size equation: step = max|X| / (2^(b-1) - 1));
    b = 4 gives [-8, 7] and step max/7, b = 8 gives [-128, 127] and step max/127."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    return -(1 << (bits - 1)), (1 << (bits - 1)) - 1


def absmax_scale(y, bits=4):
    """Unrounded per-row scale s = max(max_i |y_i| / qmax, 1e-8), float64, shape [rows];
    qmax = 7 for INT4, 127 for INT8."""
    y = np.asarray(y, dtype=np.float64)
    m = np.max(np.abs(y), axis=-1) if y.shape[-1] > 0 else np.zeros(y.shape[:-1])
    return np.maximum(m / qrange(bits)[1], SCALE_FLOOR)


def round_scale(s, dtype):
    """Round float64 scales to the storage dtype ('float32' or 'float16', RNE).

    Returns (stored values as float64, the same values in the storage dtype).
    """
    np_dtype = _SCALE_DTYPES[dtype]
    stored = np.asarray(s, dtype=np.float64).astype(np_dtype)
    return stored.astype(np.float64), stored


def quantize_codes(y, s_stored, bits=4):
    """Codes q = round_half_even(clamp(y / s, qmin, qmax)) per row, as int8 ([-8, 7] for
    INT4, [-128, 127] for INT8).

    y: [..., n] float64; s_stored: [...] float64 (the stored scale). Rows whose stored
    scale is 0 get code 0 everywhere.
    """
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(s_stored, dtype=np.float64)[..., None]
    zero = s == 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(zero, 0.0, y / np.where(zero, 1.0, s))
    lo, hi = qrange(bits)
    q = np.rint(np.clip(t, lo, hi))
    return q.astype(np.int8)


def pack_nibbles(q):
    """Two codes per byte: byte j = (q[2j] & 0xF) | ((q[2j+1] & 0xF) << 4)."""
    q = np.asarray(q, dtype=np.int64)
    if q.shape[-1] % 2:
        raise ValueError("row length must be even to pack nibbles")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(b):
    """Inverse of pack_nibbles: uint8 [..., n/2] -> int8 codes [..., n] (sign-extended)."""
    b = np.asarray(b, dtype=np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    q = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    q = np.where(q >= 8, q - 16, q)
    return q.astype(np.int8)


def dequantize(q, s_stored):
    """q * s per row, float64."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s_stored, dtype=np.float64)[..., None]


def mse(a, b):
    """Mean squared difference over all elements, float64."""
    d = np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)
    return float(np.mean(d * d)) if d.size else 0.0


def rmsnorm(h, divisor="rms"):
    """RMSNorm with its gain folded away: h / RMS(h) (or h / ||h|| with divisor='norm').

    "SpinQuant, when rotations are worth learning" (section "The math, slowly") works the
    invariance RMSNorm(R h) = R RMSNorm(h) on h = (3, 4) dividing by the length; the
    usual RMSNorm divides by the root mean square. Both divisors are rotation invariant,
    so both are offered.
    """
    h = np.asarray(h, dtype=np.float64)
    norm = np.sqrt(np.sum(h * h, axis=-1, keepdims=True))
    if divisor == "norm":
        return h / norm
    if divisor == "rms":
        return h / (norm / np.sqrt(h.shape[-1]))
    raise ValueError(divisor)


def round_to_bf16(v):
    """Round float64 values to the nearest bfloat16 (8 significant bits, ties to even),
    returned as float64. Finite, normal-range inputs only (the Q outputs it serves)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)  # v = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def hadamard_quant_int4(x, scale_dtype="float16", packed=True, rotate_input=True, signs=None, bits=4,
                        kron=False):
    """Rotate each row of x by H_n / sqrt(n), then quantize it to INT4 per row.

    x: [rows, n] (any real dtype; upcast exactly to float64).
    rotate_input=False quantizes x itself (the "without rotation" arm, and the quantizer
    for activations that already live in a rotated basis).
    signs: optional [n] vector of +-1; the rotation is then the randomized Hadamard
    H_n diag(signs) / sqrt(n) (see ``hadamard.rotate_signed``).
    bits: 4 (default) or 8 -- INT8 codes (scale max/127, range [-128, 127]) are never
    packed.
    kron: rotate by (H_m (x) H_p) / sqrt(n) (``kron.rotate_kron``), which also accepts
    row lengths that are not powers of two.

    Returns a dict with
      y        float64 [rows, n]  values that were quantized (rotated, or x itself),
      s        float64 [rows]     unrounded scales,
      scales   [rows]             stored scales in ``scale_dtype``,
      s_stored float64 [rows]     stored scales as float64,
      q        int8 [rows, n]     codes,
      codes    uint8 [rows, n/2] packed (packed=True) or int8 [rows, n] codes.
    """
    x = np.asarray(x, dtype=np.float64)
    if not rotate_input:
        y = x.copy()
    elif kron:
        y = rotate_kron(x)
    elif signs is not None:
        y = rotate_signed(x, signs)
    else:
        y = rotate(x)
    if bits == 8 and packed:
        raise ValueError("INT8 codes are stored one per byte")
    s = absmax_scale(y, bits)
    s_stored, scales = round_scale(s, scale_dtype)
    q = quantize_codes(y, s_stored, bits)
    codes = pack_nibbles(q) if packed else q
    return {"y": y, "s": s, "scales": scales, "s_stored": s_stored, "q": q, "codes": codes}


def kv_rotate_quant(q_in, k_in, scale_dtype="float16", q_rotate_only=False):
    """R3 on post-RoPE Q and K: rotate every (batch, head, token) vector over head_dim by
    H_d / sqrt(d) and quantize it to INT4 with one scale per vector, packed two per byte.

    "SpinQuant, when rotations are worth learning", section "Four rotation sites" (R3 is
    a fixed Hadamard on queries and keys after RoPE so the KV cache can be quantized).
    q_in, k_in: [B, H, S, D]. With q_rotate_only, Q is returned rotated and rounded to
    bfloat16 (as float64 values) instead of quantized.
    """
    out = {}
    for name, t in (("q", q_in), ("k", k_in)):
        t = np.asarray(t, dtype=np.float64)
        shape = t.shape
        rows = t.reshape(-1, shape[-1])
        if name == "q" and q_rotate_only:
            out["q_rot"] = round_to_bf16(rotate(rows)).reshape(shape)
            continue
        r = hadamard_quant_int4(rows, scale_dtype=scale_dtype, packed=True)
        out[name] = {
            "codes": r["codes"].reshape(shape[:-1] + (shape[-1] // 2,)),
            "q": r["q"].reshape(shape),
            "scales": r["scales"].reshape(shape[:-1]),
            "s_stored": r["s_stored"].reshape(shape[:-1]),
            "s": r["s"].reshape(shape[:-1]),
            "y": r["y"].reshape(shape),
        }
    return out


def quantize_groups(y, group, scale_dtype="float16", packed=True, bits=4):
    """Group-wise symmetric absmax quantization of rows y [rows, K]: each run of ``group``
    consecutive elements gets its own scale s = max(max|y_g| / qmax, 1e-8), stored in
    ``scale_dtype``, and codes round_half_even(clamp(y / s*, qmin, qmax)) against the
    stored scale -- the per-row quantizer of this module applied to every group
    ("SpinQuant, when rotations are worth learning": group-size 256/32 4-bit weights in
    its ExecuTorch export path; the step-size equation of "SpinQuant Guide: Learned
    Rotations for 4-Bit LLMs" per group).

    Returns a dict with s (unrounded) and s_stored (float64) [rows, K / group], scales
    (stored dtype), q int8 [rows, K] and codes (packed uint8 [rows, K/2] or int8).
    """
    y = np.asarray(y, dtype=np.float64)
    rows, k = y.shape
    if group < 1 or k % group:
        raise ValueError("the group size must divide the row length")
    g = y.reshape(rows, k // group, group)
    s = absmax_scale(g, bits)
    s_stored, scales = round_scale(s, scale_dtype)
    q = quantize_codes(g, s_stored, bits).reshape(rows, k)
    codes = pack_nibbles(q) if packed else q
    return {"s": s, "s_stored": s_stored, "scales": scales, "q": q, "codes": codes}
