"""GPU parity of hadamard_kron_quant_int4 (rows whose length is not a power of two,
rotated by the Kronecker product of a Paley matrix with a Sylvester matrix) against the
fp64 oracle, through the C ABI: element by element at small sizes, and on sampled rows
plus every-row invariants at the full down-projection width 14336 (8192 tokens)."""

import numpy as np
import pytest

import oracle
import workloads
from parity import check_quant

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rbq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_bit_quantization_fwht_amd as m

    m.lib()
    return m


def to_dev(x, dtype):
    if dtype == "float32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
        t = t.view(torch.bfloat16 if dtype == "bfloat16" else torch.float16)
    return t.cuda()


# (n, rows): Paley I and II factors of orders 12 .. 148, p from 16 to 2048; ragged row
# counts; the 32 KiB, 80 KiB and 160 KiB LDS variants
CASES = [(192, 37), (1536, 67), (2560, 41), (5120, 29), (3584, 33), (9216, 17), (6912, 19), (12288, 9),
         (13824, 7), (14336, 9), (18944, 5), (24576, 5), (28672, 3),
         # the Goethals-Seidel order 172 (11008 = 172 * 64, the GEMM workload's FFN width), and
         # Paley orders above 160 with up to eight K blocks of the MFMA
         (11008, 13), (2752, 21), (5504, 11), (2624, 9), (3136, 9), (6784, 5), (4032, 9)]


@pytest.mark.parametrize("n,rows", CASES)
@pytest.mark.parametrize("dtype", ["bfloat16", "float16", "float32"])
def test_kron_rotate_quant(rbq, n, rows, dtype):
    print(f"case hadamard_kron_quant_int4 n={n} rows={rows} dtype={dtype}", flush=True)
    assert rbq.kron_factor(n) == oracle.kron_factor(n)
    x = workloads.gen_rows(n, rows, n, dtype, kind="swiglu", n_outliers=2, factor=120)
    codes, scales, rot = rbq.hadamard_kron_quant_int4(to_dev(x, dtype), return_rotated=True)
    torch.cuda.synchronize()
    x64 = workloads.to_float64(x, dtype)
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, kron=True)
    check_quant(oracle.unpack_nibbles(codes.cpu().numpy()), scales.cpu().numpy(), ref, "float16", x64,
                y_gpu=rot.cpu().numpy())


def test_kron_unpacked_fp32_scales_strided(rbq):
    n, rows = 5120, 23
    print(f"case kron unpacked fp32 scales strided n={n}", flush=True)
    x = workloads.gen_rows(11, rows, n + 64, "bfloat16", n_outliers=1, factor=80)
    xd = to_dev(x, "bfloat16")[:, :n]
    codes, scales, rot = rbq.hadamard_kron_quant_int4(xd, packed=False, scale_dtype=torch.float32,
                                                      return_rotated=True)
    x64 = workloads.to_float64(x, "bfloat16")[:, :n]
    ref = oracle.hadamard_quant_int4(x64, "float32", packed=False, kron=True)
    check_quant(codes.cpu().numpy().view(np.int8), scales.cpu().numpy(), ref, "float32", x64,
                y_gpu=rot.cpu().numpy())


@pytest.mark.parametrize("n", [1536, 14336, 13824, 18944])
def test_kron_spikes_bit_exact(rbq, n):
    print(f"case kron spikes n={n}", flush=True)
    rows = 6
    x = np.zeros((rows, n), dtype=np.float32)
    for r in range(rows):
        x[r, (r * 7919 + 3) % n] = 60.0
    codes, scales = rbq.hadamard_kron_quant_int4(to_dev(workloads.f32_to_bf16_bits(x), "bfloat16"))
    ref = oracle.hadamard_quant_int4(x.astype(np.float64), "float16", packed=True, kron=True)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), ref["s_stored"])


def test_kron_edge_tokens_zero_rows_and_powers_of_two(rbq):
    n = 5120
    for rows in (0, 1, 2):
        print(f"case kron tokens={rows}", flush=True)
        x = workloads.gen_rows(900 + rows, max(rows, 1), n, "bfloat16")[:rows]
        codes, scales = rbq.hadamard_kron_quant_int4(to_dev(x, "bfloat16"))
        assert codes.shape == (rows, n // 2)
        if rows:
            x64 = workloads.to_float64(x, "bfloat16")
            ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, kron=True)
            check_quant(oracle.unpack_nibbles(codes.cpu().numpy()), scales.cpu().numpy(), ref, "float16", x64)
    # all-zero rows: the 1e-8 floor rounds to an fp16 zero scale, and every code is 0
    z = torch.zeros((2, n), dtype=torch.bfloat16, device="cuda")
    codes, scales = rbq.hadamard_kron_quant_int4(z)
    assert int(codes.abs().sum()) == 0
    # a power of two goes to the power-of-two path: identical results
    x = to_dev(workloads.gen_rows(5, 9, 4096, "bfloat16"), "bfloat16")
    c1, s1 = rbq.hadamard_kron_quant_int4(x)
    c2, s2 = rbq.hadamard_quant_int4(x)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


def test_kron_unsupported_lengths_raise(rbq):
    # 16640 = 65 * 256: no construction; 22016 = 172 * 128: more LDS than a workgroup has
    for n in (16640, 22016):
        x = torch.zeros((2, n), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(rbq.RBQError) as e:
            rbq.hadamard_kron_quant_int4(x)
        assert e.value.status == rbq.RBQ_ENOTSUP


def test_kron_full_size_14336(rbq):
    """Down-projection input of width 14336 = 28 * 512 (Paley II, q = 13): bf16
    [8192, 14336] with the R4 workload's recipe; sampled rows against the oracle, every row
    against the invariants, and two calls bit-identical."""
    print("case kron full size 8192x14336", flush=True)
    xbits, ch = workloads.gen_ffn(seed=0, n=14336)
    xd = to_dev(xbits, "bfloat16")
    codes, scales = rbq.hadamard_kron_quant_int4(xd)
    codes2, scales2 = rbq.hadamard_kron_quant_int4(xd)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    rows = np.unique(np.concatenate([[0, 1, 8191], np.random.default_rng(4).integers(0, 8192, 21)]))
    x64 = workloads.to_float64(xbits[rows], "bfloat16")
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, kron=True)
    c = codes.cpu().numpy()
    check_quant(oracle.unpack_nibbles(c[rows]), scales.cpu().numpy()[rows], ref, "float16", x64)
    q_all = oracle.unpack_nibbles(c)
    assert np.all(np.max(np.abs(q_all), axis=1) == 7)
    assert not np.any(q_all == -8)


def test_kron_full_size_11008(rbq):
    """FFN width 11008 = 172 * 64 (the Goethals-Seidel factor), bf16 [8192, 11008] with the
    R4 workload's recipe: sampled rows against the oracle, every row against the
    invariants, two calls bit-identical."""
    print("case kron full size 8192x11008", flush=True)
    assert rbq.kron_factor(11008) == 172
    xbits, ch = workloads.gen_ffn(seed=0, n=11008)
    xd = to_dev(xbits, "bfloat16")
    codes, scales = rbq.hadamard_kron_quant_int4(xd)
    codes2, scales2 = rbq.hadamard_kron_quant_int4(xd)
    torch.cuda.synchronize()
    assert torch.equal(codes, codes2) and torch.equal(scales, scales2)
    rows = np.unique(np.concatenate([[0, 1, 8191], np.random.default_rng(7).integers(0, 8192, 29)]))
    x64 = workloads.to_float64(xbits[rows], "bfloat16")
    ref = oracle.hadamard_quant_int4(x64, "float16", packed=False, kron=True)
    c = codes.cpu().numpy()
    check_quant(oracle.unpack_nibbles(c[rows]), scales.cpu().numpy()[rows], ref, "float16", x64)
    q_all = oracle.unpack_nibbles(c)
    assert np.all(np.max(np.abs(q_all), axis=1) == 7)
    assert not np.any(q_all == -8)
