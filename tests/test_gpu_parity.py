"""GPU parity of the fused Hadamard + INT4 quantizer (hadamard_quant_int4) and the R3
per-head op (kv_rotate_quant) against the fp64 oracle, through the C ABI.

Small cases are checked element by element; the full workload sizes, in the launch
configuration the benchmark times, are checked on sampled rows the oracle computes one
by one plus properties that hold for every row.
"""

import math

import numpy as np
import pytest

import oracle
import workloads
from parity import check_quant, check_rope_quant, check_rope_rotated

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rbq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_bit_quantization_fwht_amd as m

    m.lib()  # raises if the library is missing: no fallback
    return m


def to_dev(x, dtype):
    if dtype == "float32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
        t = t.view(torch.bfloat16 if dtype == "bfloat16" else torch.float16)
    return t.cuda()


def unpack(codes_dev):
    return oracle.unpack_nibbles(codes_dev.cpu().numpy())


ROWS = {1: 8200, 2: 4100, 3: 2050, 4: 1030, 5: 515, 6: 260, 7: 131, 8: 70, 9: 35, 10: 17, 11: 9, 12: 5,
        13: 3, 14: 3, 15: 2}


@pytest.mark.parametrize("k", list(range(1, 16)))
@pytest.mark.parametrize("dtype", ["bfloat16", "float32", "float16"])
def test_rotate_quant_all_sizes(rbq, k, dtype):
    n, rows = 1 << k, ROWS[k]
    print(f"case hadamard_quant_int4 k={k} dtype={dtype} rows={rows}", flush=True)
    x = workloads.gen_rows(k, rows, n, dtype, kind="swiglu", n_outliers=1, factor=150)
    codes, scales, rot = rbq.hadamard_quant_int4(to_dev(x, dtype), return_rotated=True)
    torch.cuda.synchronize()
    x64 = workloads.to_float64(x, dtype)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    check_quant(unpack(codes), scales.cpu().numpy(), ref, "float16", x64, y_gpu=rot.cpu().numpy())


@pytest.mark.parametrize("signed", [False, True])
@pytest.mark.parametrize("k", list(range(1, 16)))
@pytest.mark.parametrize("dtype", ["bfloat16", "float16", "float32"])
def test_codes_only_all_sizes(rbq, k, dtype, signed):
    """The default call: packed codes and fp16 scales with no rotated output. For 16-bit
    inputs this is its own kernel build (codes-only, with its own register budget and
    waves per SIMD), the one the benchmark times; every row length, with and without the
    randomized diagonal, element by element against the oracle."""
    n, rows = 1 << k, ROWS[k]
    print(f"case codes-only k={k} dtype={dtype} signed={signed} rows={rows}", flush=True)
    x = workloads.gen_rows(300 + k, rows, n, dtype, kind="swiglu", n_outliers=2, factor=150)
    xd = to_dev(x, dtype)
    x64 = workloads.to_float64(x, dtype)
    if signed:
        s32 = workloads.gen_signs(k + 40, n)
        sd = torch.from_numpy(s32).to("cuda").to({"float32": torch.float32, "bfloat16": torch.bfloat16,
                                                 "float16": torch.float16}[dtype])
        ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, signs=s32)
        codes, scales = rbq.hadamard_quant_int4(xd, signs=sd)
    else:
        ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
        codes, scales = rbq.hadamard_quant_int4(xd)
    torch.cuda.synchronize()
    check_quant(unpack(codes), scales.cpu().numpy(), ref, "float16", x64)


@pytest.mark.parametrize("k", [1, 4, 7, 12, 14, 15])
def test_no_rotate_exact(rbq, k):
    n, rows = 1 << k, ROWS[k]
    print(f"case no-rotate k={k}", flush=True)
    x = workloads.gen_rows(100 + k, rows, n, "bfloat16", n_outliers=1, factor=60)
    codes, scales, rot = rbq.hadamard_quant_int4(to_dev(x, "bfloat16"), rotate=False, return_rotated=True)
    x64 = workloads.to_float64(x, "bfloat16")
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, rotate_input=False)
    st = check_quant(unpack(codes), scales.cpu().numpy(), ref, "float16", x64, rotate=False, y_gpu=rot.cpu().numpy())
    assert st["code_flips"] == 0


def test_edge_token_counts(rbq):
    for k in (7, 12, 14):
        n = 1 << k
        for rows in (0, 1, 3):
            print(f"case tokens={rows} k={k}", flush=True)
            x = workloads.gen_rows(500 + rows, max(rows, 1), n, "bfloat16")[:rows]
            codes, scales = rbq.hadamard_quant_int4(to_dev(x, "bfloat16"))
            torch.cuda.synchronize()
            assert codes.shape == (rows, n // 2)
            if rows:
                x64 = workloads.to_float64(x, "bfloat16")
                ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
                check_quant(unpack(codes), scales.cpu().numpy(), ref, "float16", x64)


def test_strided_rows_and_output_bounds(rbq):
    k, n = 12, 4096
    full = workloads.gen_rows(9, 33, n + 128, "bfloat16", n_outliers=2, factor=90)
    xd = to_dev(full, "bfloat16")[:, :n]
    assert xd.stride(0) == n + 128
    # guard bytes around the outputs must stay untouched
    codes_buf = torch.full((33 * n // 2 + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    codes = codes_buf[:33 * n // 2].view(33, n // 2)
    codes, scales = rbq.hadamard_quant_int4(xd, codes=codes)
    torch.cuda.synchronize()
    assert torch.all(codes_buf[33 * n // 2:] == 0xA5)
    x64 = workloads.to_float64(full[:, :n], "bfloat16")
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    check_quant(unpack(codes), scales.cpu().numpy(), ref, "float16", x64)


def test_spike_bit_exact(rbq):
    n, ch = 4096, 142
    x = np.zeros((3, n), dtype=np.float32)
    x[0, ch] = 60.0
    x[1, ch] = -60.0
    codes, scales, rot = rbq.hadamard_quant_int4(to_dev(x, "float32"), return_rotated=True)
    ref = oracle.hadamard_quant_int4(x.astype(np.float64), "float16", packed=True)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), ref["s_stored"])
    assert np.array_equal(rot.cpu().numpy().astype(np.float64), ref["y"])


def test_worked_example_config_full(rbq):
    """64 x 4096 fp32, channel 142 = 60: int8 codes + fp32 scales, and the MSE of the
    dequantized result with and without rotation."""
    print("case worked example 64x4096", flush=True)
    x = workloads.gen_worked_example(seed=0)
    xd = to_dev(x, "float32")
    codes, scales, rot = rbq.hadamard_quant_int4(xd, scale_dtype=torch.float32, packed=False, return_rotated=True)
    dcodes, dscales = rbq.hadamard_quant_int4(xd, scale_dtype=torch.float32, packed=False, rotate=False)
    x64 = x.astype(np.float64)
    ref = oracle.hadamard_quant_int4(x64, "float32", packed=False)
    check_quant(codes.cpu().numpy(), scales.cpu().numpy(), ref, "float32", x64, y_gpu=rot.cpu().numpy())
    dref = oracle.hadamard_quant_int4(x64, "float32", packed=False, rotate_input=False)
    st = check_quant(dcodes.cpu().numpy(), dscales.cpu().numpy(), dref, "float32", x64, rotate=False)
    assert st["code_flips"] == 0
    # MSE from the GPU outputs vs from the oracle (dequantize + rotate back on the host)
    q, s = codes.cpu().numpy().astype(np.float64), scales.cpu().numpy().astype(np.float64)
    mse_gpu = oracle.mse(x64, oracle.rotate(q * s[:, None]))
    mse_ref = oracle.mse(x64, oracle.rotate(oracle.dequantize(ref["q"], ref["s_stored"])))
    dq, ds = dcodes.cpu().numpy().astype(np.float64), dscales.cpu().numpy().astype(np.float64)
    mse_direct_gpu = oracle.mse(x64, dq * ds[:, None])
    mse_direct_ref = oracle.mse(x64, oracle.dequantize(dref["q"], dref["s_stored"]))
    assert abs(mse_gpu / mse_ref - 1) < 1e-3
    assert abs(mse_direct_gpu / mse_direct_ref - 1) < 1e-3
    assert mse_gpu < 0.1 * mse_direct_gpu


def test_ffn_config_full_size(rbq):
    """R4 at the full workload: bf16 [8192, 16384], packed codes, fp16 scales; sampled rows
    against the oracle, every row against the invariants."""
    print("case R4 full size 8192x16384", flush=True)
    xbits, ch = workloads.gen_ffn(seed=0)
    xd = to_dev(xbits, "bfloat16")
    codes, scales = rbq.hadamard_quant_int4(xd)
    codes2, scales2 = rbq.hadamard_quant_int4(xd)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)  # deterministic
    rows = np.unique(np.concatenate([[0, 1, 8191], np.random.default_rng(3).integers(0, 8192, 29)]))
    x64 = workloads.to_float64(xbits[rows], "bfloat16")
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    c = codes.cpu().numpy()
    check_quant(oracle.unpack_nibbles(c[rows]), scales.cpu().numpy()[rows], ref, "float16", x64)
    # every row: the absmax element lands on +-7, no code is -8, the scale is positive
    q_all = oracle.unpack_nibbles(c)
    assert np.all(np.max(np.abs(q_all), axis=1) == 7)
    assert not np.any(q_all == -8)
    assert np.all(scales.cpu().numpy().astype(np.float64) > 0)


@pytest.mark.parametrize("tokens", workloads.DECODE_TOKENS)
@pytest.mark.parametrize("n", workloads.DECODE_N)
def test_decode_sweep_points(rbq, tokens, n):
    print(f"case decode T={tokens} n={n}", flush=True)
    xbits, _ = workloads.gen_decode(seed=0, tokens=tokens, n=n)
    codes, scales = rbq.hadamard_quant_int4(to_dev(xbits, "bfloat16"))
    sample = np.arange(tokens) if tokens * n <= 64 * 8192 else np.unique(np.linspace(0, tokens - 1, 8).astype(int))
    x64 = workloads.to_float64(xbits[sample], "bfloat16")
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    check_quant(unpack(codes)[sample], scales.cpu().numpy()[sample], ref, "float16", x64)


# ------------------------------------------------------------------ R3: kv_rotate_quant


@pytest.mark.parametrize("layout", ["contiguous", "bshd_view"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_kv_small(rbq, layout, D):
    B, H, S = 2, 3, 45
    print(f"case kv small D={D} layout={layout}", flush=True)
    q_bits, k_bits, _ = workloads.gen_kv(seed=D, batch=B, heads=H, seq=S, head_dim=D)
    if layout == "contiguous":
        qd, kd = to_dev(q_bits, "bfloat16"), to_dev(k_bits, "bfloat16")
    else:
        qd = to_dev(np.ascontiguousarray(q_bits.transpose(0, 2, 1, 3)), "bfloat16").permute(0, 2, 1, 3)
        kd = to_dev(np.ascontiguousarray(k_bits.transpose(0, 2, 1, 3)), "bfloat16").permute(0, 2, 1, 3)
    out = rbq.kv_rotate_quant(qd, kd)
    ref = oracle.kv_rotate_quant(workloads.to_float64(q_bits, "bfloat16"), workloads.to_float64(k_bits, "bfloat16"))
    for name in ("q", "k"):
        rows = B * H * S
        x64 = workloads.to_float64(q_bits if name == "q" else k_bits, "bfloat16").reshape(rows, D)
        r = {key: ref[name][key].reshape(rows, -1) if ref[name][key].ndim == 4 else ref[name][key].reshape(rows)
             for key in ("y", "q", "s", "s_stored")}
        got_q = oracle.unpack_nibbles(out[f"{name}_codes"].cpu().numpy().reshape(rows, D // 2))
        check_quant(got_q, out[f"{name}_scales"].cpu().numpy().reshape(rows), r, "float16", x64)


def test_kv_q_rotate_only(rbq):
    B, H, S, D = 1, 4, 33, 128
    q_bits, k_bits, _ = workloads.gen_kv(seed=1, batch=B, heads=H, seq=S, head_dim=D)
    out = rbq.kv_rotate_quant(to_dev(q_bits, "bfloat16"), to_dev(k_bits, "bfloat16"), q_rotate_only=True)
    got = out["q_rotated"].float().cpu().numpy().astype(np.float64)
    want = oracle.round_to_bf16(oracle.rotate(workloads.to_float64(q_bits, "bfloat16")))
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7)
    assert np.mean(got == want) > 0.999
    rows = B * H * S
    x64 = workloads.to_float64(k_bits, "bfloat16").reshape(rows, D)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
    check_quant(oracle.unpack_nibbles(out["k_codes"].cpu().numpy().reshape(rows, D // 2)),
                out["k_scales"].cpu().numpy().reshape(rows), ref, "float16", x64)


def test_kv_config_full_size(rbq):
    """R3 at the full workload: Q and K [16, 32, 2048, 128] bf16 in one call."""
    print("case R3 full size", flush=True)
    q_bits, k_bits, ch = workloads.gen_kv(seed=0)
    qd, kd = to_dev(q_bits, "bfloat16"), to_dev(k_bits, "bfloat16")
    out = rbq.kv_rotate_quant(qd, kd)
    out2 = rbq.kv_rotate_quant(qd, kd)
    torch.cuda.synchronize()
    for key in out:
        assert torch.equal(out[key], out2[key])
    rows_all = 16 * 32 * 2048
    sample = np.unique(np.concatenate([[0, rows_all - 1], np.random.default_rng(4).integers(0, rows_all, 4000)]))
    for name, bits in (("q", q_bits), ("k", k_bits)):
        x64 = workloads.to_float64(bits.reshape(rows_all, 128)[sample], "bfloat16")
        ref = oracle.hadamard_quant_int4(x64, "float16", packed=False)
        c = out[f"{name}_codes"].view(rows_all, 64).cpu().numpy()
        s = out[f"{name}_scales"].view(rows_all).cpu().numpy()
        check_quant(oracle.unpack_nibbles(c[sample]), s[sample], ref, "float16", x64)
        q_all = oracle.unpack_nibbles(c[::97])
        assert np.all(np.max(np.abs(q_all), axis=1) == 7) and not np.any(q_all == -8)


def test_binding_rejects_bad_output_buffers(rbq):
    """Caller-provided outputs of the wrong shape, dtype or layout are refused before any
    launch (the kernels write them without bounds checks)."""
    x = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        rbq.hadamard_quant_int4(x, codes=torch.empty((8, 64), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        rbq.hadamard_quant_int4(x, codes=torch.empty((8, 128), dtype=torch.int8, device="cuda"))
    with pytest.raises(ValueError):
        rbq.hadamard_quant_int4(x, scales=torch.empty((7,), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        rbq.hadamard_quant_int4(x, codes=torch.empty((128, 8), dtype=torch.uint8, device="cuda").t())
    q = torch.zeros((1, 2, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        rbq.kv_rotate_quant(q, q.clone(), k_codes=torch.empty((1, 2, 4, 32), dtype=torch.uint8, device="cuda"))
    qa = torch.zeros((4, 64), dtype=torch.uint8, device="cuda")
    sa = torch.ones((4,), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        rbq.w4a4_gemm(qa, sa, qa, sa, out=torch.empty((4, 3), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        rbq.w4a4_gemm(qa, sa, qa, sa[:3])


@pytest.mark.parametrize("k,dtype", [(1, "float32"), (3, "bfloat16"), (7, "bfloat16"), (9, "float16"),
                                     (12, "float32"), (14, "bfloat16"), (15, "float16")])
def test_randomized_rotation(rbq, k, dtype):
    """H diag(signs) / sqrt(n) through hadamard_quant_int4_signed: codes-only launches and
    launches that also return the rotated rows, against the oracle's randomized transform."""
    n = 1 << k
    rows = max(3, min(300, (1 << 16) // n))
    print(f"case randomized k={k} {dtype} rows={rows}", flush=True)
    x = workloads.gen_rows(50 + k, rows, n, dtype, kind="swiglu", n_outliers=3, factor=120)
    s32 = workloads.gen_signs(k, n)
    sd = torch.from_numpy(s32).to("cuda").to({"float32": torch.float32, "bfloat16": torch.bfloat16,
                                             "float16": torch.float16}[dtype])
    xd = to_dev(x, dtype)
    x64 = workloads.to_float64(x, dtype)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, signs=s32)
    codes, scales = rbq.hadamard_quant_int4(xd, signs=sd)
    check_quant(oracle.unpack_nibbles(codes.cpu().numpy()), scales.cpu().numpy(), ref, "float16", x64)
    codes, scales, rot = rbq.hadamard_quant_int4(xd, signs=sd, return_rotated=True)
    check_quant(oracle.unpack_nibbles(codes.cpu().numpy()), scales.cpu().numpy(), ref, "float16", x64,
                y_gpu=rot.cpu().numpy())
    with pytest.raises(rbq.RBQError):
        rbq.hadamard_quant_int4(xd, signs=sd, rotate=False)


@pytest.mark.parametrize("k,dtype,rot", [(3, "float32", True), (7, "bfloat16", True), (10, "float16", True),
                                         (12, "bfloat16", True), (14, "bfloat16", True), (15, "float32", True),
                                         (12, "bfloat16", False)])
def test_int8_codes(rbq, k, dtype, rot):
    """hadamard_quant_int8: scale max/127, codes in [-128, 127] one per byte."""
    n = 1 << k
    rows = max(3, min(300, (1 << 16) // n))
    print(f"case int8 k={k} {dtype} rot={rot} rows={rows}", flush=True)
    x = workloads.gen_rows(90 + k, rows, n, dtype, kind="swiglu", n_outliers=3, factor=120)
    xd = to_dev(x, dtype)
    x64 = workloads.to_float64(x, dtype)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, rotate_input=rot, bits=8)
    codes, scales, y = rbq.hadamard_quant_int8(xd, rotate=rot, return_rotated=True)
    st = check_quant(codes.cpu().numpy(), scales.cpu().numpy(), ref, "float16", x64, rotate=rot,
                     y_gpu=y.cpu().numpy(), bits=8)
    if not rot:
        assert st["code_flips"] == 0
    codes2, scales2 = rbq.hadamard_quant_int8(xd, rotate=rot)
    assert torch.equal(codes2, codes) and torch.equal(scales2, scales)


def rope_tables(positions, d, base=10000.0):
    inv = base ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)
    th = np.outer(np.arange(positions, dtype=np.float64), inv)
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


@pytest.mark.parametrize("dtype,layout,pos0,bhs", [
    ("bfloat16", "contiguous", 0, (2, 3, 45)), ("bfloat16", "bshd_view", 7, (2, 3, 45)),
    ("float16", "contiguous", 100, (2, 3, 45)), ("float16", "bshd_view", 0, (2, 3, 45)),
    # shapes whose rows fill whole 64-row blocks, several blocks per workgroup loop
    ("bfloat16", "contiguous", 3, (2, 6, 80)), ("bfloat16", "bshd_view", 0, (4, 5, 48)),
    ("float16", "contiguous", 0, (1, 4, 16)), ("float16", "bshd_view", 9, (8, 2, 272)),
    # head-group order (heads a multiple of 4, tokens of 16; for head_dim 256 of 8 and 8)
    ("bfloat16", "contiguous", 5, (2, 8, 48)), ("float16", "bshd_view", 0, (3, 16, 32))])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_kv_rope_small(rbq, dtype, layout, pos0, bhs, D):
    """kv_rope_rotate_quant: RoPE (half-split; the oracle evaluates it exactly and rounds it
    once to the 16-bit format, accepting the other neighbour only where float32 evaluation
    error reaches a rounding midpoint) then R3 and INT4, on Q and K."""
    B, H, S = bhs
    print(f"case kv rope D={D} {dtype} {layout} pos0={pos0} B,H,S={bhs}", flush=True)
    q_bits, k_bits, _ = workloads.gen_kv(seed=17, batch=B, heads=H, seq=S, head_dim=D)
    if dtype == "float16":
        q_bits = workloads.bf16_bits_to_f32(q_bits).astype(np.float16).view(np.uint16)
        k_bits = workloads.bf16_bits_to_f32(k_bits).astype(np.float16).view(np.uint16)
    if layout == "contiguous":
        qd, kd = to_dev(q_bits, dtype), to_dev(k_bits, dtype)
    else:
        qd = to_dev(np.ascontiguousarray(q_bits.transpose(0, 2, 1, 3)), dtype).permute(0, 2, 1, 3)
        kd = to_dev(np.ascontiguousarray(k_bits.transpose(0, 2, 1, 3)), dtype).permute(0, 2, 1, 3)
    cos, sin = rope_tables(pos0 + S, D)
    out = rbq.kv_rotate_quant(qd, kd, rope_cos=torch.from_numpy(cos).cuda(), rope_sin=torch.from_numpy(sin).cuda(),
                              rope_pos0=pos0)
    pos = pos0 + np.arange(S)
    rows = B * H * S
    cr = np.broadcast_to(cos[pos][None, None], (B, H, S, D // 2)).reshape(rows, D // 2)
    sr = np.broadcast_to(sin[pos][None, None], (B, H, S, D // 2)).reshape(rows, D // 2)
    for name, bits in (("q", q_bits), ("k", k_bits)):
        x16 = workloads.to_float64(bits, dtype).reshape(rows, D)
        got_q = oracle.unpack_nibbles(out[f"{name}_codes"].cpu().numpy().reshape(rows, D // 2))
        st = check_rope_quant(got_q, out[f"{name}_scales"].cpu().numpy().reshape(rows), x16, cr, sr, dtype)
        print(f"  {name}: {st}", flush=True)


@pytest.mark.parametrize("bhs", [(1, 3, 37), (2, 2, 64), (2, 8, 32)])
def test_kv_rope_q_rotate_only(rbq, bhs):
    """RoPE + R3 with Q written rotated in bf16 (no codes): each rotated row lands at its
    own (batch, head, token) place, with a ragged last block, with whole blocks, and with
    blocks in head-group order."""
    B, H, S = bhs
    D = 128
    print(f"case kv rope q_rotate_only B,H,S={bhs}", flush=True)
    q_bits, k_bits, _ = workloads.gen_kv(seed=23, batch=B, heads=H, seq=S, head_dim=D)
    cos, sin = rope_tables(S + 2, D)
    out = rbq.kv_rotate_quant(to_dev(q_bits, "bfloat16"), to_dev(k_bits, "bfloat16"), q_rotate_only=True,
                              rope_cos=torch.from_numpy(cos).cuda(), rope_sin=torch.from_numpy(sin).cuda(),
                              rope_pos0=2)
    pos = 2 + np.arange(S)
    rows = B * H * S
    cr = np.broadcast_to(cos[pos][None, None], (B, H, S, D // 2)).reshape(rows, D // 2)
    sr = np.broadcast_to(sin[pos][None, None], (B, H, S, D // 2)).reshape(rows, D // 2)
    got = out["q_rotated"].float().cpu().numpy().astype(np.float64).reshape(rows, D)
    check_rope_rotated(got, workloads.to_float64(q_bits, "bfloat16").reshape(rows, D), cr, sr, "bfloat16")
    check_rope_quant(oracle.unpack_nibbles(out["k_codes"].cpu().numpy().reshape(rows, D // 2)),
                     out["k_scales"].cpu().numpy().reshape(rows),
                     workloads.to_float64(k_bits, "bfloat16").reshape(rows, D), cr, sr, "bfloat16")


def test_kv_rope_full_size_and_errors(rbq):
    """The fused RoPE + R3 at the full R3 workload (sampled rows against the oracle, all
    rows against the invariants), and the argument checks."""
    print("case kv rope full size", flush=True)
    B, H, S, D = 16, 32, 2048, 128
    q_bits, k_bits, _ = workloads.gen_kv(seed=2)
    cos, sin = rope_tables(S + 64, D)
    cd, sd = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    qd, kd = to_dev(q_bits, "bfloat16"), to_dev(k_bits, "bfloat16")
    out = rbq.kv_rotate_quant(qd, kd, rope_cos=cd, rope_sin=sd, rope_pos0=64)
    rng = np.random.default_rng(5)
    flat = rng.integers(0, B * H * S, 40)
    b, h, s = flat // (H * S), (flat // S) % H, flat % S
    kc = out["k_codes"].cpu().numpy().reshape(B * H * S, D // 2)[flat]
    ks = out["k_scales"].cpu().numpy().reshape(B * H * S)[flat]
    check_rope_quant(oracle.unpack_nibbles(kc), ks, workloads.to_float64(k_bits[b, h, s], "bfloat16"),
                     cos[64 + s], sin[64 + s], "bfloat16")
    qa = oracle.unpack_nibbles(out["q_codes"].cpu().numpy().reshape(B * H * S, D // 2))
    assert np.all(np.max(np.abs(qa), axis=1) == 7) and not np.any(qa == -8)
    with pytest.raises(rbq.RBQError):   # tables too short for rope_pos0 + seq
        rbq.kv_rotate_quant(qd, kd, rope_cos=cd, rope_sin=sd, rope_pos0=65)
    q32 = torch.zeros((1, 1, 4, 32), dtype=torch.bfloat16, device="cuda")
    c32 = torch.zeros((8, 16), dtype=torch.float32, device="cuda")
    with pytest.raises(rbq.RBQError):   # head_dim 32 is not fused (64, 128 and 256 are)
        rbq.kv_rotate_quant(q32, q32.clone(), rope_cos=c32, rope_sin=c32)
