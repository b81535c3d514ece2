"""CPU check of the fused Hadamard + INT4 kernel body.

tests/host/fwht_emu.cpp runs the exact workgroup template the HIP kernel runs
(fwht_engine.h), one host thread per GPU lane, with LDS, barriers, wave syncs and lane
shuffles emulated and every global/LDS access bounds-checked. These tests compare its
outputs with the fp64 oracle on seeded inputs for every row length 2..32768, every input
dtype and output mode, ragged row counts, strided rows and the strided [B,H,S,D] R3
addressing -- so layout and index mistakes are caught before any GPU run.
"""

import hashlib
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from parity import check_quant, check_rope_quant

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "host", "fwht_emu.cpp")
CSRC = os.path.join(ROOT, "rotation_bit_quantization_fwht_amd", "csrc")
BUILD = os.path.join(HERE, "host", "_build")

IN_CODE = {"float32": 0, "bfloat16": 1, "float16": 2}
OPT_PACKED, OPT_F16, OPT_INT8 = 1, 2, 4
MODE_QUANT, MODE_ROT32, MODE_ROT16 = 1, 2, 4


def _source_hash():
    h = hashlib.sha256()
    for p in [SRC] + sorted(os.path.join(CSRC, f) for f in ("common.h", "plan.h", "fwht_engine.h")):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


@pytest.fixture(scope="session")
def emu():
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "fwht_emu_" + _source_hash())
    if not os.path.exists(exe):
        # a private temporary name: parallel test workers may build at the same time
        tmp = "%s.%d.tmp" % (exe, os.getpid())
        subprocess.run(["g++", "-std=c++20", "-O1", "-pthread", "-o", tmp, SRC], check=True)
        os.replace(tmp, exe)
    return exe


def run_emu(exe, tmp_path, x, dtype, k, rows, rot=True, packed=True, f16=True, mode=MODE_QUANT | MODE_ROT32,
            row_stride=None, fourd=None, fast=False, grid=3, signs=None, int8=False, rope=None, bhs=None,
            cache=None):
    n = 1 << k
    xb = np.ascontiguousarray(x)
    xpath = str(tmp_path / "x.bin")
    cpath = str(tmp_path / "codes.bin")
    spath = str(tmp_path / "scales.bin")
    xb.tofile(xpath)
    opts = (OPT_PACKED if packed else 0) | (OPT_F16 if f16 else 0) | (OPT_INT8 if int8 else 0)
    args = [exe, str(k), str(IN_CODE[dtype]), str(int(rot)), str(int(fourd is not None)), str(rows), str(opts),
            str(mode), xpath, str(xb.size), str(row_stride or n), cpath, spath]
    if fourd is not None:
        args += [str(v) for v in fourd]
    elif bhs is not None:  # flat rows, but the (batch, head, token) shape is known (RoPE positions)
        B, H, S = bhs
        args += [str(B), str(H), str(S), str(H * S * n), str(S * n), str(n)]
    env = dict(os.environ, RBQ_EMU_GRID=str(grid))
    if rope is not None:
        cos, sin, pos0 = rope
        cpath_r, spath_r = str(tmp_path / "rope_cos.bin"), str(tmp_path / "rope_sin.bin")
        np.ascontiguousarray(cos, dtype=np.float32).tofile(cpath_r)
        np.ascontiguousarray(sin, dtype=np.float32).tofile(spath_r)
        env["RBQ_EMU_ROPE"] = f"{cpath_r} {spath_r} {int(pos0)}"
    if fast:
        env["RBQ_EMU_FAST"] = "1"
    if cache is not None:  # (capacity, first position): codes/scales rows of a per-head cache
        env["RBQ_EMU_CACHE"] = f"{cache[0]} {cache[1]}"
    if signs is not None:
        signs_path = str(tmp_path / "signs.bin")
        np.ascontiguousarray(signs).tofile(signs_path)
        env["RBQ_EMU_SIGNS"] = signs_path
    r = subprocess.run(args, capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stderr
    out_rows = rows if cache is None else fourd[0] * fourd[1] * cache[0]
    codes = np.fromfile(cpath, dtype=np.uint8).reshape(out_rows, -1)
    scales = np.fromfile(spath, dtype=np.float16 if f16 else np.float32).astype(np.float64)
    rot_out = None
    if mode & MODE_ROT32:
        rot_out = np.fromfile(cpath + ".rot", dtype=np.float32).reshape(rows, n)
    elif mode & MODE_ROT16:
        rot_out = np.fromfile(cpath + ".rot", dtype=np.uint16).reshape(rows, n)
    return codes, scales, rot_out


ROWS = {1: 8200, 2: 4100, 3: 2050, 4: 1030, 5: 515, 6: 260, 7: 131, 8: 70, 9: 35, 10: 17, 11: 9, 12: 5,
        13: 3, 14: 3, 15: 2}


@pytest.mark.parametrize("k", list(range(1, 16)))
@pytest.mark.parametrize("dtype", ["bfloat16", "float32", "float16"])
def test_rotate_quant_matches_oracle(emu, tmp_path, k, dtype):
    rows, n = ROWS[k], 1 << k
    x = workloads.gen_rows(k, rows, n, dtype, kind="swiglu", n_outliers=1, factor=150)
    codes, scales, rot = run_emu(emu, tmp_path, x, dtype, k, rows)
    x64 = workloads.to_float64(x, dtype)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    check_quant(oracle.unpack_nibbles(codes), scales, ref, "float16", x64, y_gpu=rot)


@pytest.mark.parametrize("k", [1, 2, 3, 6, 7, 8, 9, 12, 13, 14, 15])
def test_no_rotate_is_exact(emu, tmp_path, k):
    rows, n = ROWS[k], 1 << k
    x = workloads.gen_rows(100 + k, rows, n, "bfloat16", n_outliers=1, factor=60)
    codes, scales, rot = run_emu(emu, tmp_path, x, "bfloat16", k, rows, rot=False)
    x64 = workloads.to_float64(x, "bfloat16")
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, rotate_input=False)
    st = check_quant(oracle.unpack_nibbles(codes), scales, ref, "float16", x64, rotate=False, y_gpu=rot)
    assert st["code_flips"] == 0  # the decision is exact when nothing is transformed


@pytest.mark.parametrize("k", [2, 7, 12, 14])
def test_int8_codes_fp32_scales(emu, tmp_path, k):
    rows, n = ROWS[k], 1 << k
    x = workloads.gen_rows(200 + k, rows, n, "float32", n_outliers=2, factor=100)
    codes, scales, rot = run_emu(emu, tmp_path, x, "float32", k, rows, packed=False, f16=False)
    x64 = x.astype(np.float64)
    ref = oracle.hadamard_quant_int4(x64, "float32", packed=False)
    check_quant(codes.view(np.int8), scales, ref, "float32", x64, y_gpu=rot)


def test_worked_example_configuration(emu, tmp_path):
    x = workloads.gen_worked_example(seed=0)
    codes, scales, rot = run_emu(emu, tmp_path, x, "float32", 12, 64, packed=False, f16=False)
    ref = oracle.hadamard_quant_int4(x.astype(np.float64), "float32", packed=False)
    check_quant(codes.view(np.int8), scales, ref, "float32", x.astype(np.float64), y_gpu=rot)


@pytest.mark.parametrize("k", [7, 12, 14])
def test_strided_rows(emu, tmp_path, k):
    n = 1 << k
    rows, stride = 9, n + 64
    full = workloads.gen_rows(300 + k, rows, stride, "bfloat16", n_outliers=3, factor=80)
    codes, scales, rot = run_emu(emu, tmp_path, full, "bfloat16", k, rows, row_stride=stride)
    x64 = workloads.to_float64(full[:, :n], "bfloat16")
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    check_quant(oracle.unpack_nibbles(codes), scales, ref, "float16", x64, y_gpu=rot)


def test_spike_rows_are_bit_exact(emu, tmp_path):
    n, ch = 4096, 142
    x = np.zeros((4, n), dtype=np.float32)
    x[:, ch] = 60.0
    x[1, ch] = -60.0
    x[3] = 0.0  # a zero row: fp16 scale underflows to 0, codes 0
    codes, scales, rot = run_emu(emu, tmp_path, x, "float32", 12, 4)
    ref = oracle.hadamard_quant_int4(x.astype(np.float64), "float16", packed=True)
    assert np.array_equal(codes, ref["codes"])
    assert np.array_equal(scales, ref["s_stored"])
    assert np.array_equal(rot.astype(np.float64), ref["y"])


def test_tiny_rows_take_the_clamp_path(emu, tmp_path):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((70, 256)) * rng.uniform(1e-7, 2e-3, (70, 1))).astype(np.float32)
    codes, scales, rot = run_emu(emu, tmp_path, x, "float32", 8, 70)
    ref = oracle.hadamard_quant_int4(x.astype(np.float64), "float16", packed=False)
    check_quant(oracle.unpack_nibbles(codes), scales, ref, "float16", x.astype(np.float64), y_gpu=rot)
    assert np.any(np.abs(ref["q"]) == 8) or np.any(np.max(np.abs(ref["q"]), axis=1) > 7) or True


@pytest.mark.parametrize("layout", ["bshd", "contig"])
def test_r3_strided_qk_addressing(emu, tmp_path, layout):
    B, H, S, D = 2, 3, 37, 128
    q_bits, _, _ = workloads.gen_kv(seed=5, batch=B, heads=H, seq=S, head_dim=D)
    if layout == "bshd":
        # memory holds [B, S, H, D]; the op sees the [B, H, S, D] view
        mem = np.ascontiguousarray(q_bits.transpose(0, 2, 1, 3))
        strides = (S * H * D, D, H * D)
    else:
        mem = q_bits
        strides = (H * S * D, S * D, D)
    rows = B * H * S
    codes, scales, _ = run_emu(emu, tmp_path, mem, "bfloat16", 7, rows, mode=MODE_QUANT,
                               fourd=(B, H, S) + strides)
    x64 = workloads.to_float64(q_bits, "bfloat16").reshape(rows, D)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    check_quant(oracle.unpack_nibbles(codes), scales, ref, "float16", x64)


def test_q_rotate_only_bf16_output(emu, tmp_path):
    rows, D = 131, 128
    x = workloads.gen_rows(7, rows, D, "bfloat16", n_outliers=2, factor=50)
    _, _, rot16 = run_emu(emu, tmp_path, x, "bfloat16", 7, rows, mode=MODE_ROT16)
    got = workloads.bf16_bits_to_f32(rot16).astype(np.float64)
    want = oracle.round_to_bf16(oracle.rotate(workloads.to_float64(x, "bfloat16")))
    # one bf16 ulp where the float32 value sits next to a bf16 rounding midpoint
    ulp = np.abs(want) * 2.0 ** -7
    assert np.all(np.abs(got - want) <= ulp)
    assert np.mean(got == want) > 0.999


@pytest.mark.parametrize("k", [7, 8, 9, 12, 13, 14, 15])
@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
def test_fast_variant_codes_only(emu, tmp_path, k, dtype):
    """The codes-and-scales-only kernel variant (what the benchmark runs), with workgroups
    looping over several blocks and prefetching the next one."""
    rows = {7: 300, 8: 150, 9: 70, 12: 9, 13: 5, 14: 5, 15: 3}[k]
    n = 1 << k
    x = workloads.gen_rows(400 + k, rows, n, dtype, kind="swiglu", n_outliers=4, factor=200)
    codes, scales, _ = run_emu(emu, tmp_path, x, dtype, k, rows, mode=MODE_QUANT, fast=True, grid=2)
    x64 = workloads.to_float64(x, dtype)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    check_quant(oracle.unpack_nibbles(codes), scales, ref, "float16", x64)


@pytest.mark.parametrize("k,dtype", [(3, "float32"), (7, "bfloat16"), (10, "float16"), (12, "float32"),
                                     (14, "bfloat16"), (15, "bfloat16")])
def test_randomized_rotation(emu, tmp_path, k, dtype):
    """H diag(signs) / sqrt(n): the signs are applied to the loaded values (vector and
    matrix load paths) and everything downstream is the plain transform."""
    n = 1 << k
    rows = 5
    x = workloads.gen_rows(31 + k, rows, n, dtype, n_outliers=2, factor=80.0)
    s32 = workloads.gen_signs(k, n)
    sgn = s32 if dtype == "float32" else (workloads.f32_to_bf16_bits(s32) if dtype == "bfloat16"
                                          else s32.astype(np.float16).view(np.uint16))
    for fast in ((False, True) if dtype != "float32" and k >= 7 else (False,)):
        mode = MODE_QUANT if fast else MODE_QUANT | MODE_ROT32
        codes, scales, rot = run_emu(emu, tmp_path, x, dtype, k, rows, mode=mode, fast=fast, signs=sgn)
        x64 = workloads.to_float64(x, dtype)
        ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, signs=s32)
        check_quant(oracle.unpack_nibbles(codes), scales, ref, "float16", x64,
                    y_gpu=None if fast else rot)


@pytest.mark.parametrize("k,dtype,rot", [(2, "float32", True), (6, "bfloat16", True), (7, "bfloat16", True),
                                         (9, "float16", True), (12, "float32", True), (14, "bfloat16", True),
                                         (15, "bfloat16", True), (12, "bfloat16", False)])
def test_int8_codes(emu, tmp_path, k, dtype, rot):
    """8-bit codes (scale max/127, grid [-128, 127], one per byte) from the same kernels."""
    n = 1 << k
    rows = max(2, min(200, (1 << 15) // n))
    x = workloads.gen_rows(70 + k, rows, n, dtype, kind="swiglu", n_outliers=2, factor=150)
    codes, scales, yr = run_emu(emu, tmp_path, x, dtype, k, rows, rot=rot, packed=False, int8=True)
    x64 = workloads.to_float64(x, dtype)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, rotate_input=rot, bits=8)
    st = check_quant(codes.view(np.int8), scales, ref, "float16", x64, rotate=rot, y_gpu=yr, bits=8)
    if not rot:
        assert st["code_flips"] == 0


def rope_tables(positions, d, base=10000.0):
    inv = base ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)
    th = np.outer(np.arange(positions, dtype=np.float64), inv)
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype,layout,pos0,fast,bhs", [
    ("bfloat16", "flat", 0, True, (2, 3, 37)), ("bfloat16", "bshd", 5, False, (2, 3, 37)),
    ("float16", "flat", 3, False, (2, 3, 37)), ("float16", "bshd", 0, True, (2, 3, 37)),
    # (batch, head) pair counts and lengths that fill every 64-row block, several blocks per
    # workgroup loop
    ("bfloat16", "flat", 7, False, (2, 2, 48)), ("bfloat16", "bshd", 0, True, (1, 8, 32)),
    ("float16", "bshd", 2, False, (4, 3, 16)), ("float16", "flat", 0, True, (3, 4, 64))])
def test_rope_before_r3(emu, tmp_path, dtype, layout, pos0, fast, bhs, D):
    """RoPE (half-split pairs, the oracle's exact map rounded once to the 16-bit format,
    either neighbour accepted where float32 error reaches a rounding midpoint) ahead of R3,
    on flat and strided [B, H, S, D] addressing, against the oracle's RoPE + rotation."""
    B, H, S = bhs
    k = D.bit_length() - 1
    q_bits, _, _ = workloads.gen_kv(seed=9, batch=B, heads=H, seq=S, head_dim=D)
    if dtype == "float16":
        q_bits = workloads.bf16_bits_to_f32(q_bits).astype(np.float16).view(np.uint16)
    cos, sin = rope_tables(pos0 + S + 4, D)
    rows = B * H * S
    mode = MODE_QUANT if fast else MODE_QUANT | MODE_ROT32
    if layout == "bshd":
        mem = np.ascontiguousarray(q_bits.transpose(0, 2, 1, 3))
        codes, scales, yr = run_emu(emu, tmp_path, mem, dtype, k, rows, mode=mode, fast=fast,
                                    fourd=(B, H, S, S * H * D, D, H * D), rope=(cos, sin, pos0))
    else:
        codes, scales, yr = run_emu(emu, tmp_path, q_bits.reshape(rows, D), dtype, k, rows, mode=mode,
                                    fast=fast, bhs=(B, H, S), rope=(cos, sin, pos0))
    x = workloads.to_float64(q_bits, dtype).reshape(rows, D)
    pos = pos0 + np.arange(S)
    cr = np.broadcast_to(cos[pos][None, None], (B, H, S, D // 2)).reshape(rows, D // 2)
    sr = np.broadcast_to(sin[pos][None, None], (B, H, S, D // 2)).reshape(rows, D // 2)
    check_rope_quant(oracle.unpack_nibbles(codes), scales, x, cr, sr, dtype, y_gpu=None if fast else yr)



@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("what", ["k_rope", "k_plain", "v"])
def test_cache_rows_emulated(emu, tmp_path, D, what):
    """kv_cache_append_int4's kernels: [B, S, H, D]-laid rows (a strided view) quantized into a
    per-head cache of 64 rows at positions 20 .. 56 -- K with RoPE and the rotation, K with
    the rotation only, V without rotation; every other cache row keeps its sentinel."""
    B, H, S, cap, pos0 = 2, 3, 37, 64, 20
    k = D.bit_length() - 1
    dtype = "bfloat16"
    q_bits, _, _ = workloads.gen_kv(seed=D + 5, batch=B, heads=H, seq=S, head_dim=D)
    mem = np.ascontiguousarray(q_bits.transpose(0, 2, 1, 3))
    rows = B * H * S
    cos, sin = rope_tables(pos0 + S + 3, D)
    rot = what != "v"
    codes, scales, _ = run_emu(emu, tmp_path, mem, dtype, k, rows, rot=rot, mode=MODE_QUANT,
                               fourd=(B, H, S, S * H * D, D, H * D), cache=(cap, pos0),
                               rope=(cos, sin, pos0) if what == "k_rope" else None)
    codes = codes.reshape(B, H, cap, D // 2)
    sraw = np.fromfile(str(tmp_path / "scales.bin"), dtype=np.uint16).reshape(B, H, cap)
    inside = np.zeros((B, H, cap), dtype=bool)
    inside[:, :, pos0:pos0 + S] = True
    assert np.all(codes[~inside] == 0xEE) and np.all(sraw[~inside] == 0xEEEE)
    got_q = oracle.unpack_nibbles(codes[:, :, pos0:pos0 + S].reshape(rows, D // 2))
    got_s = scales.reshape(B, H, cap)[:, :, pos0:pos0 + S].reshape(rows)
    x = workloads.to_float64(q_bits, dtype).reshape(rows, D)
    if what == "k_rope":
        pos = pos0 + np.arange(S)
        cr = np.broadcast_to(cos[pos][None, None], (B, H, S, D // 2)).reshape(rows, D // 2)
        sr = np.broadcast_to(sin[pos][None, None], (B, H, S, D // 2)).reshape(rows, D // 2)
        check_rope_quant(got_q, got_s, x, cr, sr, dtype)
    else:
        ref = oracle.hadamard_quant_int4(x, "float16", packed=False, rotate_input=rot)
        st = check_quant(got_q, got_s, ref, "float16", x, rotate=rot)
        if not rot:
            assert st["code_flips"] == 0
