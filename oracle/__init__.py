"""Plain fp64 CPU oracle for online Hadamard rotation + symmetric INT4 quantization
and the W4A4 integer GEMM that consumes the codes.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with the HIP library (no kernels, headers,
tables, helpers or pre/post-processing); the only module both sides read is the
seeded input generator ``workloads.py``, which holds none of the method's arithmetic.

Everything is computed in float64 with NumPy, following the definitions on the pages:

* ``hadamard``: the Sylvester construction of H_n and the rotation y = H_n x / sqrt(n)
  as an explicit matrix product ("Rotations: QuaRot, SpinQuant and incoherence",
  section "Hadamard matrices").
* ``quant``: per-row symmetric absmax INT4 quantization, scale = max|y| / 7, clamp to
  [-8, 7] and round half to even ("SpinQuant Guide: Learned Rotations for 4-Bit LLMs",
  the outlier-curse figure, the step-size equation and the ``uniform_quantize_int4``
  listing), nibble packing, dequantization and MSE.
* ``gemm``: exact integer product of the codes and the scale epilogue.
* ``rope``: the rotary position embedding that the fused R3 operation applies first.
* ``kron``: rotations of rows whose length is not a power of two, by the Kronecker
  product of a Paley matrix with a Sylvester matrix.
* ``attention``: decode attention over the INT4 key/value cache.

Every function here is pinned by ``tests/test_oracle.py`` against facts the pages or
the mathematics fix (worked examples, closed forms, invariants, brute force); a
function without such a pin says "parity unpinned" in its docstring.
"""

from .hadamard import sylvester, hadamard_popcount, hadamard_column_block, rotate, rotate_signed
from .quant import (
    SCALE_FLOOR,
    qrange,
    QMIN,
    QMAX,
    absmax_scale,
    round_scale,
    quantize_codes,
    pack_nibbles,
    unpack_nibbles,
    dequantize,
    mse,
    rmsnorm,
    round_to_bf16,
    hadamard_quant_int4,
    kv_rotate_quant,
    quantize_groups,
)
from .gemm import int_gemm, w4a4_gemm, w4a8_gemm, w4a8_gemm_grouped
from .rope import rope_exact, rope_16bit, rope_16bit_ambiguous, round_to_format
from .attention import attention_decode
from .kron import (legendre, paley_kind, paley_hadamard, kron_factor, kron_hadamard, rotate_kron,
                   gs_first_rows, goethals_seidel_hadamard, small_hadamard, periodic_autocorrelation)

__all__ = [
    "sylvester",
    "hadamard_popcount",
    "hadamard_column_block",
    "rotate",
    "rotate_signed",
    "qrange",
    "SCALE_FLOOR",
    "QMIN",
    "QMAX",
    "absmax_scale",
    "round_scale",
    "quantize_codes",
    "pack_nibbles",
    "unpack_nibbles",
    "dequantize",
    "mse",
    "rmsnorm",
    "round_to_bf16",
    "hadamard_quant_int4",
    "kv_rotate_quant",
    "int_gemm",
    "w4a4_gemm",
    "w4a8_gemm",
    "w4a8_gemm_grouped",
    "quantize_groups",
    "rope_exact",
    "rope_16bit",
    "rope_16bit_ambiguous",
    "round_to_format",
    "legendre",
    "paley_kind",
    "paley_hadamard",
    "kron_factor",
    "kron_hadamard",
    "rotate_kron",
    "gs_first_rows",
    "goethals_seidel_hadamard",
    "small_hadamard",
    "periodic_autocorrelation",
    "attention_decode",
]
