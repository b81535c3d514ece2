"""CPU check of the rotation + INT4 kernel for row lengths that are not powers of two.

tests/host/kron_emu.cpp runs the workgroup template of kron_engine.h (the code the HIP
kernel runs) with one host thread per GPU lane, emulated LDS, barriers, shuffles and
MFMAs, and every access bounds-checked; its kernel arguments come from the library's own
host logic (kron_factor.h). Outputs are compared with the fp64 oracle's
(H_m (x) H_p) / sqrt(n) rotation and quantizer.
"""

import hashlib
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from parity import check_quant

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "host", "kron_emu.cpp")
CSRC = os.path.join(ROOT, "rotation_bit_quantization_fwht_amd", "csrc")
BUILD = os.path.join(HERE, "host", "_build")
IN_CODE = {"float32": 0, "bfloat16": 1, "float16": 2}


def _source_hash():
    h = hashlib.sha256()
    for p in [SRC, os.path.join(HERE, "host", "host_ctx.h")] + sorted(
            os.path.join(CSRC, f) for f in ("common.h", "plan.h", "fwht_engine.h", "kron_engine.h", "kron_factor.h")):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


@pytest.fixture(scope="session")
def kemu():
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "kron_emu_" + _source_hash())
    if not os.path.exists(exe):
        tmp = "%s.%d.tmp" % (exe, os.getpid())
        subprocess.run(["g++", "-std=c++20", "-O1", "-pthread", "-o", tmp, SRC], check=True)
        os.replace(tmp, exe)
    return exe


def run_kemu(exe, tmp_path, x, dtype, n, rows, packed=True, f16=True, rot=True, row_stride=None, grid=2):
    xpath, cpath, spath, rpath = (str(tmp_path / f) for f in ("x.bin", "codes.bin", "scales.bin", "rot.bin"))
    np.ascontiguousarray(x).tofile(xpath)
    opts = (1 if packed else 0) | (2 if f16 else 0)
    args = [exe, str(IN_CODE[dtype]), str(n), str(rows), str(opts), xpath, str(row_stride or n), cpath, spath]
    if rot:
        args.append(rpath)
    r = subprocess.run(args, capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, RBQ_EMU_GRID=str(grid)))
    assert r.returncode == 0, r.stderr
    m, p, paley, q, words = (int(v) for v in r.stdout.split())
    codes = np.fromfile(cpath, dtype=np.uint8).reshape(rows, -1)
    scales = np.fromfile(spath, dtype=np.float16 if f16 else np.float32).astype(np.float64)
    y = np.fromfile(rpath, dtype=np.float32).reshape(rows, n) if rot else None
    return codes, scales, y, (m, p, paley, q)


# (n, rows): every Paley kind, p from 16 to 2048, one to three passes of butterflies; the
# Goethals-Seidel order 172 (11008 = 172 * 64, 2752 = 172 * 16) and Paley orders above 160
# (164, 196 of the second kind, 212, 252: up to eight K blocks of the MFMA)
CASES = [(192, 5), (1536, 3), (2560, 3), (5120, 3), (3584, 3), (9216, 2), (6912, 2), (12288, 2),
         (18944, 2), (24576, 2), (28672, 1), (11008, 2), (2752, 3), (2624, 2), (3136, 2), (6784, 1),
         (4032, 2)]


@pytest.mark.parametrize("n,rows", CASES)
@pytest.mark.parametrize("dtype", ["bfloat16", "float16", "float32"])
def test_kron_rotate_quant_matches_oracle(kemu, tmp_path, n, rows, dtype):
    x = workloads.gen_rows(n, rows, n, dtype, kind="swiglu", n_outliers=2, factor=120)
    codes, scales, y, (m, p, paley, q) = run_kemu(kemu, tmp_path, x, dtype, n, rows)
    assert m == oracle.kron_factor(n) and m * p == n
    assert (q, paley) == (oracle.paley_kind(m) or (43, 3))  # kind 3: the Goethals-Seidel order 172
    x64 = workloads.to_float64(x, dtype)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, kron=True)
    check_quant(oracle.unpack_nibbles(codes), scales, ref, "float16", x64, y_gpu=y)


def test_kron_unpacked_codes_fp32_scales_strided_rows(kemu, tmp_path):
    n, rows, stride = 5120, 3, 5120 + 24
    x = workloads.gen_rows(7, rows, stride, "bfloat16", n_outliers=1, factor=80)
    codes, scales, y, _ = run_kemu(kemu, tmp_path, x, "bfloat16", n, rows, packed=False, f16=False,
                                   row_stride=stride)
    x64 = workloads.to_float64(x, "bfloat16")[:, :n]
    ref = oracle.hadamard_quant_int4(x64, "float32", packed=False, kron=True)
    check_quant(codes.view(np.int8), scales, ref, "float32", x64, y_gpu=y)


@pytest.mark.parametrize("n", [1536, 14336, 13824])
def test_kron_spike_rows_bit_exact(kemu, tmp_path, n):
    # a spike maps to a +-1 column of H_m (x) H_p: every |y| equals 60 / sqrt(n) and every
    # code is +-7, so codes and scales must match the oracle exactly
    rows = 3
    x = np.zeros((rows, n), dtype=np.float32)
    for r in range(rows):
        x[r, (r * 977 + 5) % n] = 60.0
    xb = workloads.f32_to_bf16_bits(x)
    codes, scales, y, _ = run_kemu(kemu, tmp_path, xb, "bfloat16", n, rows)
    ref = oracle.hadamard_quant_int4(x.astype(np.float64), "float16", packed=True, kron=True)
    assert np.array_equal(codes, ref["codes"])
    assert np.array_equal(scales, ref["s_stored"])
    assert np.all(np.abs(oracle.unpack_nibbles(codes)) == 7)


def test_kron_rejects_unsupported_lengths(kemu, tmp_path):
    # 16640 = 65 * 256: no construction of order 260 or below; 22016 = 172 * 128: the
    # row buffer and the operand table exceed a workgroup's LDS
    for n in (16640, 22016):
        x = np.zeros((1, n), dtype=np.uint16)
        xpath = str(tmp_path / "x.bin")
        x.tofile(xpath)
        r = subprocess.run([kemu, "1", str(n), "1", "1", xpath, str(n), str(tmp_path / "c"), str(tmp_path / "s")],
                           capture_output=True, text=True, timeout=60)
        assert r.returncode == 3, n
