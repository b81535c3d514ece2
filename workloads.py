"""Seeded synthetic inputs for the online-rotation hot path.

This is the only module that both the HIP path's tests/bench and the fp64 oracle read.
It draws random numbers and converts them to the storage formats the kernels consume
(float32, bfloat16 bit patterns); it holds none of the method's arithmetic (no
rotation, scaling, rounding-to-code or packing).

The workloads stand in for LLaMA-class activations (the pages evaluate on WikiText-2 and
zero-shot suites, which are not used here): Gaussian values with a few persistent
outlier channels, the pattern described in "SpinQuant Guide: Learned Rotations for
4-Bit LLMs" (section "The Emergence of Emergent Activation Outliers": a small set of
channels 100-200x the typical magnitude) and in the worked example of "Rotations:
QuaRot, SpinQuant and incoherence" (one channel at 60 among 4096 near +-1).

All draws use ``numpy.random.default_rng`` with an explicit seed, in the order written
in each generator, as float32; bfloat16 inputs are the float32 draws rounded to nearest
even on the bit pattern.
"""

import numpy as np

# ---------------------------------------------------------------------------------
# Storage-format helpers (format conversion only).
# ---------------------------------------------------------------------------------


def f32_to_bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even (finite)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key):
    return np.random.default_rng([int(k) for k in key])


def _silu(a):
    return a / (np.float32(1.0) + np.exp(-a))


# ---------------------------------------------------------------------------------
# The five workloads. Default sizes are the full configurations; every generator also
# takes smaller sizes for parity tests.
# ---------------------------------------------------------------------------------

WORKLOADS = {
    1: "worked example: fp32 [64, 4096], N(0,1), channel 142 set to 60.0",
    2: "R3 KV path: bf16 Q and K [16, 32, 2048, 128], N(0,1), 2 seeded head_dim channels x50",
    3: "R4 FFN path: bf16 [8192, 16384] = silu(a)*b, a,b ~ N(0,1), 8 seeded channels x200",
    4: "decode sweep: bf16 [T, n], T in {1,4,16,64,256}, n in {4096,8192,32768}, one channel x100",
    5: "W4A4 GEMM: A bf16 [4096, 4096] N(0,1) + one channel x60; W fp32 [11008, 4096] N(0, 0.02^2)",
}

DECODE_TOKENS = (1, 4, 16, 64, 256)
DECODE_N = (4096, 8192, 32768)


def gen_worked_example(seed=0, tokens=64, n=4096, channel=142, value=60.0):
    """Workload 1: x ~ N(0,1) float32 [tokens, n], then x[:, channel] = value."""
    x = _rng(seed, 1).standard_normal((tokens, n), dtype=np.float32)
    if n > channel:
        x[:, channel] = np.float32(value)
    return x


def gen_kv(seed=0, batch=16, heads=32, seq=2048, head_dim=128, n_outliers=2, factor=50.0):
    """Workload 2: post-RoPE Q and K, each [B, H, S, D] as bfloat16 bit patterns.

    Draw order: Q values, K values (float32 N(0,1)), then ``n_outliers`` distinct
    head_dim channels; those channels of both Q and K are multiplied by ``factor``.
    Returns (q_bits, k_bits, channels).
    """
    rng = _rng(seed, 2)
    shape = (batch, heads, seq, head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    ch = np.sort(rng.choice(head_dim, size=min(n_outliers, head_dim), replace=False))
    q[..., ch] *= np.float32(factor)
    k[..., ch] *= np.float32(factor)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), ch


def gen_ffn(seed=0, tokens=8192, n=16384, n_outliers=8, factor=200.0):
    """Workload 3: down_proj input silu(a) * b, [tokens, n] as bfloat16 bit patterns.

    Draw order: a, b (float32 N(0,1)), then ``n_outliers`` distinct channels that are
    multiplied by ``factor`` in every token. Returns (x_bits, channels).
    """
    rng = _rng(seed, 3)
    a = rng.standard_normal((tokens, n), dtype=np.float32)
    b = rng.standard_normal((tokens, n), dtype=np.float32)
    x = _silu(a)
    del a
    x *= b
    del b
    ch = np.sort(rng.choice(n, size=min(n_outliers, n), replace=False))
    x[:, ch] *= np.float32(factor)
    return f32_to_bf16_bits(x), ch


def gen_decode(seed=0, tokens=1, n=4096, factor=100.0):
    """Workload 4 point (tokens, n): N(0,1) [tokens, n], one seeded channel x factor,
    as bfloat16 bit patterns. Returns (x_bits, channel)."""
    rng = _rng(seed, 4, tokens, n)
    x = rng.standard_normal((tokens, n), dtype=np.float32)
    ch = int(rng.integers(0, n))
    x[:, ch] *= np.float32(factor)
    return f32_to_bf16_bits(x), ch


def gen_gemm_inputs(seed=0, m=4096, n=11008, k=4096, factor=60.0, w_std=0.02):
    """Workload 5 raw inputs: activation A [m, k] (bfloat16 bits; N(0,1) with one seeded
    channel x factor) and weight W [n, k] (float32, N(0, w_std^2)).

    Draw order: A values, the outlier channel, W values. Returns (a_bits, w, channel).
    """
    rng = _rng(seed, 5)
    a = rng.standard_normal((m, k), dtype=np.float32)
    ch = int(rng.integers(0, k))
    a[:, ch] *= np.float32(factor)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(w_std)
    return f32_to_bf16_bits(a), w, ch


def gen_rows(seed, rows, n, dtype="bfloat16", n_outliers=1, factor=100.0, kind="normal"):
    """Generic rows for parity sweeps: N(0,1) (kind='normal') or silu(a)*b
    (kind='swiglu') with ``n_outliers`` seeded channels x factor.

    dtype 'float32' returns float32 values; 'bfloat16' / 'float16' return uint16 bit
    patterns (bfloat16 rounded to nearest even; float16 via numpy's RNE cast).
    """
    rng = _rng(seed, 6, rows, n)
    if kind == "swiglu":
        a = rng.standard_normal((rows, n), dtype=np.float32)
        b = rng.standard_normal((rows, n), dtype=np.float32)
        x = _silu(a) * b
    else:
        x = rng.standard_normal((rows, n), dtype=np.float32)
    if n_outliers and n > 0:
        ch = rng.choice(n, size=min(n_outliers, n), replace=False)
        x[:, ch] *= np.float32(factor)
    if dtype == "float32":
        return x
    if dtype == "bfloat16":
        return f32_to_bf16_bits(x)
    if dtype == "float16":
        return x.astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def to_float64(x, dtype):
    """Exact float64 view of an input produced above ('float32', 'bfloat16', 'float16')."""
    if dtype == "float32":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bfloat16":
        return bf16_bits_to_f32(x).astype(np.float64)
    if dtype == "float16":
        return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def gen_packed_codes(seed, rows, k):
    """Uniformly random packed INT4 codes: uint8 [rows, k/2], every nibble value -8..7
    equally likely (stand-in operands for GEMM tests at any size)."""
    return _rng(seed, 7, rows, k).integers(0, 256, size=(rows, k // 2), dtype=np.uint8)


def gen_scales(seed, n, dtype="float16", lo=1e-3, hi=0.1):
    """Positive per-row scales, log-uniform in [lo, hi], in the storage dtype."""
    v = np.exp(_rng(seed, 8, n).uniform(np.log(lo), np.log(hi), size=n))
    return v.astype(np.float16 if dtype == "float16" else np.float32)


def gen_signs(seed, n):
    """A seeded random +-1 diagonal of length n (float32), for the randomized Hadamard."""
    return np.where(_rng(seed, 9, n).integers(0, 2, size=n) == 1, 1.0, -1.0).astype(np.float32)
