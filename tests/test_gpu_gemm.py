"""GPU parity of w4a4_gemm against the oracle's exact integer GEMM, through the C ABI:
int32 accumulators bit-exact, bf16 outputs within 1e-2 relative. Operands are oracle-made
codes of the rotated workload (small sizes) or seeded random packed codes (any size)."""

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rbq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_bit_quantization_fwht_amd as m

    m.lib()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_out(acc_gpu, out_gpu, acc_ref, sa, sw):
    assert np.array_equal(acc_gpu.astype(np.int64), acc_ref), "int32 accumulators differ"
    ref = acc_ref.astype(np.float64) * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    got = out_gpu.astype(np.float64)
    zero = acc_ref == 0
    assert np.all(got[zero] == 0.0)
    rel = np.abs(got[~zero] - ref[~zero]) / np.abs(ref[~zero])
    assert rel.size == 0 or float(rel.max()) <= 1e-2, f"bf16 output rel err {rel.max():.3g}"


def run(rbq, qa, sa, qw, sw):
    out, acc = rbq.w4a4_gemm(dev(qa), dev(sa), dev(qw), dev(sw), return_acc=True)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.float().cpu().numpy()


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (64, 256, 128), (300, 264, 1024), (256, 512, 4096),
                                   (513, 1032, 2048), (77, 11008 // 43, 4096)])
@pytest.mark.parametrize("sdt", ["float16", "float32"])
def test_gemm_random_codes(rbq, M, N, K, sdt):
    print(f"case w4a4_gemm M={M} N={N} K={K} scales={sdt}", flush=True)
    qa = workloads.gen_packed_codes(1, M, K)
    qw = workloads.gen_packed_codes(2, N, K)
    sa = workloads.gen_scales(3, M, sdt)
    sw = workloads.gen_scales(4, N, sdt)
    acc, out = run(rbq, qa, sa, qw, sw)
    acc_ref = oracle.int_gemm(oracle.unpack_nibbles(qa), oracle.unpack_nibbles(qw))
    check_out(acc, out, acc_ref, sa, sw)


def test_gemm_extreme_codes(rbq):
    # all codes -8: the largest magnitude sum, 64 * K per output
    M, N, K = 64, 64, 65536
    qa = np.full((M, K // 2), 0x88, dtype=np.uint8)
    qw = np.full((N, K // 2), 0x88, dtype=np.uint8)
    s = np.ones(M, dtype=np.float16)
    acc, out = run(rbq, qa, s, qw, s[:N])
    assert np.all(acc == 64 * K)


def test_gemm_on_rotated_workload_codes(rbq):
    """The path end to end at reduced size: rotated, quantized activations and weights."""
    ab, w, _ = workloads.gen_gemm_inputs(seed=3, m=96, n=264, k=2048)
    ra = oracle.hadamard_quant_int4(workloads.to_float64(ab, "bfloat16"), "float16", packed=True)
    rw = oracle.hadamard_quant_int4(w.astype(np.float64), "float16", packed=True)
    acc, out = run(rbq, ra["codes"], ra["scales"], rw["codes"], rw["scales"])
    acc_ref, _ = oracle.w4a4_gemm(ra["q"], ra["s_stored"], rw["q"], rw["s_stored"])
    check_out(acc, out, acc_ref, ra["s_stored"], rw["s_stored"])


def test_gemm_full_size_sampled(rbq):
    """The full workload shape, M=4096, N=11008, K=4096: sampled rows exactly, and row and
    column sums of every accumulator against identities computable at any size."""
    M, N, K = 4096, 11008, 4096
    print("case w4a4_gemm full size", flush=True)
    qa = workloads.gen_packed_codes(11, M, K)
    qw = workloads.gen_packed_codes(12, N, K)
    sa = workloads.gen_scales(13, M)
    sw = workloads.gen_scales(14, N)
    acc, out = run(rbq, qa, sa, qw, sw)
    a_codes = oracle.unpack_nibbles(qa).astype(np.int64)
    w_codes = oracle.unpack_nibbles(qw).astype(np.int64)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(5).integers(0, M, 28)]))
    acc_ref = oracle.int_gemm(a_codes[rows], w_codes)
    check_out(acc[rows], out[rows], acc_ref, sa[rows], sw)
    # sum over n of acc[m, n] = a[m] . (sum_n w[n]);  sum over m = (sum_m a[m]) . w[n]
    assert np.array_equal(acc.astype(np.int64).sum(axis=1), a_codes @ w_codes.sum(axis=0))
    assert np.array_equal(acc.astype(np.int64).sum(axis=0), w_codes @ a_codes.sum(axis=0))


def test_gemm_full_size_rotated_workload(rbq):
    """The GEMM workload end to end at its full shape, M=4096, N=11008, K=4096, on the
    oracle's codes of the rotated workload (A: bf16 activations with an outlier channel x60,
    W: fp32 N(0, 0.02^2) weights, both rotated by H_4096 / 64 and quantized per row):
    sampled rows exactly, every accumulator through its row and column sums."""
    M, N, K = 4096, 11008, 4096
    print("case w4a4_gemm full size on rotated workload codes (oracle quantizes A and W)", flush=True)
    ab, w, _ = workloads.gen_gemm_inputs(seed=0)
    ra = oracle.hadamard_quant_int4(workloads.to_float64(ab, "bfloat16"), "float16", packed=True)
    del ab
    rw = oracle.hadamard_quant_int4(w.astype(np.float64), "float16", packed=True)
    del w
    print("case w4a4_gemm full size: oracle codes ready, launching", flush=True)
    acc, out = run(rbq, ra["codes"], ra["scales"], rw["codes"], rw["scales"])
    a_codes = ra["q"].astype(np.int64)
    w_codes = rw["q"].astype(np.int64)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(6).integers(0, M, 28)]))
    acc_ref = oracle.int_gemm(a_codes[rows], w_codes)
    check_out(acc[rows], out[rows], acc_ref, ra["s_stored"][rows], rw["s_stored"])
    assert np.array_equal(acc.astype(np.int64).sum(axis=1), a_codes @ w_codes.sum(axis=0))
    assert np.array_equal(acc.astype(np.int64).sum(axis=0), w_codes @ a_codes.sum(axis=0))


# ------------------------------------------------------------------------------ W4A8

def gen_int8_codes(seed, rows, k):
    """Uniform INT8 activation codes in [-127, 127] (what the quantizer can produce)."""
    return np.random.default_rng([seed, 11, rows, k]).integers(-127, 128, size=(rows, k)).astype(np.int8)


def run8(rbq, qa, sa, qw, sw):
    out, acc = rbq.w4a8_gemm(dev(qa), dev(sa), dev(qw), dev(sw), return_acc=True)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.float().cpu().numpy()


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (64, 256, 128), (300, 264, 1024), (256, 512, 4096),
                                   (513, 1032, 2048)])
def test_w4a8_random_codes(rbq, M, N, K):
    print(f"case w4a8_gemm M={M} N={N} K={K}", flush=True)
    qa = gen_int8_codes(1, M, K)
    qw = workloads.gen_packed_codes(2, N, K)
    sa = workloads.gen_scales(3, M, "float16")
    sw = workloads.gen_scales(4, N, "float16")
    acc, out = run8(rbq, qa, sa, qw, sw)
    acc_ref, _ = oracle.w4a8_gemm(qa, sa, oracle.unpack_nibbles(qw), sw)
    check_out(acc, out, acc_ref, sa, sw)


# Tile grids that exercise the workgroup -> tile order of the 256 x 256 kernels: tile counts
# that are multiples of 8 (each XCD given an eighth of the sequence) with the last group of
# 8 tile columns 1, 4 or 5 wide, ragged M and N, and a count that is not (plain order).
TILE_GRIDS = [(2048, 2304, 256), (1024, 5120, 128), (1800, 2056, 128), (2048, 3328, 256), (1280, 4352, 128)]


@pytest.mark.parametrize("M,N,K", TILE_GRIDS)
@pytest.mark.parametrize("which", ["w4a4", "w4a8"])
def test_gemm_tile_grids_exact(rbq, M, N, K, which):
    print(f"case {which} tile grid M={M} N={N} K={K} tiles={-(-M // 256)}x{-(-N // 256)}", flush=True)
    qw = workloads.gen_packed_codes(2, N, K)
    sa = workloads.gen_scales(3, M, "float16")
    sw = workloads.gen_scales(4, N, "float16")
    if which == "w4a4":
        qa = workloads.gen_packed_codes(1, M, K)
        acc, out = run(rbq, qa, sa, qw, sw)
        acc_ref = oracle.int_gemm(oracle.unpack_nibbles(qa), oracle.unpack_nibbles(qw))
    else:
        qa = gen_int8_codes(1, M, K)
        acc, out = run8(rbq, qa, sa, qw, sw)
        acc_ref, _ = oracle.w4a8_gemm(qa, sa, oracle.unpack_nibbles(qw), sw)
    check_out(acc, out, acc_ref, sa, sw)


def test_w4a8_extreme_codes(rbq):
    """-128 x -8 everywhere at the largest supported K: the sums reach 1024 * 65536 = 2^26
    (2^30 with the kernel's factor 16) and must stay exact."""
    M, N, K = 32, 64, 65536
    print("case w4a8_gemm extremes K=65536", flush=True)
    qa = np.full((M, K), -128, dtype=np.int8)
    qa[1::2, ::3] = 127
    qw = np.full((N, K // 2), 0x88, dtype=np.uint8)  # every nibble -8
    sa = np.ones(M, dtype=np.float32)
    sw = np.ones(N, dtype=np.float32)
    acc, out = run8(rbq, qa, sa, qw, sw)
    acc_ref, _ = oracle.w4a8_gemm(qa, sa, oracle.unpack_nibbles(qw), sw)
    check_out(acc, out, acc_ref, sa, sw)


def test_w4a8_on_int8_quantized_workload(rbq):
    """The W4A8 pipeline end to end on the GEMM workload's shapes (reduced M): A rotated and
    quantized to INT8 by hadamard_quant_int8, W to INT4 by hadamard_quant_int4."""
    M, N, K = 256, 1024, 4096
    print("case w4a8 pipeline 256x1024x4096", flush=True)
    ab, w, _ = workloads.gen_gemm_inputs(seed=3, m=M, n=N, k=K)
    a_d = torch.from_numpy(np.ascontiguousarray(ab).view(np.int16)).view(torch.bfloat16).cuda()
    qa, sa = rbq.hadamard_quant_int8(a_d)
    qw, sw = rbq.hadamard_quant_int4(torch.from_numpy(w).cuda())
    out, acc = rbq.w4a8_gemm(qa, sa, qw, sw, return_acc=True)
    torch.cuda.synchronize()
    qa_h, sa_h = qa.cpu().numpy(), sa.cpu().numpy()
    qw_h, sw_h = oracle.unpack_nibbles(qw.cpu().numpy()), sw.cpu().numpy()
    acc_ref, _ = oracle.w4a8_gemm(qa_h, sa_h, qw_h, sw_h)
    check_out(acc.cpu().numpy(), out.float().cpu().numpy(), acc_ref, sa_h, sw_h)


@pytest.mark.parametrize("which", ["w4a4", "w4a8"])
def test_gemm_bitwise_deterministic(rbq, which):
    """Integer sums and a fixed epilogue order: repeated calls on the same operands give
    bit-identical accumulators and outputs (full 4096 x 11008 x 4096 shape)."""
    M, N, K = 4096, 11008, 4096
    print(f"case {which}_gemm determinism M={M} N={N} K={K}", flush=True)
    if which == "w4a4":
        qa = dev(workloads.gen_packed_codes(41, M, K))
        call = rbq.w4a4_gemm
    else:
        qa = dev(gen_int8_codes(41, M, K))
        call = rbq.w4a8_gemm
    qw = dev(workloads.gen_packed_codes(42, N, K))
    sa = dev(workloads.gen_scales(43, M, "float16"))
    sw = dev(workloads.gen_scales(44, N, "float16"))
    runs = [call(qa, sa, qw, sw, return_acc=True) for _ in range(3)]
    torch.cuda.synchronize()
    for out, acc in runs[1:]:
        assert torch.equal(acc, runs[0][1])
        assert torch.equal(out.view(torch.int16), runs[0][0].view(torch.int16))


# Few tokens (M <= 64, decode): the kernel that streams the weights once, one workgroup per
# 32 weight rows with the waves splitting K. Ragged N (not a multiple of 32), K from one
# 128-code block to the FFN width, one and two 32-token blocks.
SMALL_M = [(1, 11008, 4096), (5, 136, 128), (31, 264, 4096), (32, 8, 128), (33, 520, 2048),
           (64, 11008, 256), (17, 4104, 14336)]


@pytest.mark.parametrize("M,N,K", SMALL_M)
def test_gemm_few_tokens(rbq, M, N, K):
    print(f"case w4a4_gemm few tokens M={M} N={N} K={K}", flush=True)
    qa = workloads.gen_packed_codes(5, M, K)
    qw = workloads.gen_packed_codes(6, N, K)
    sa = workloads.gen_scales(7, M, "float16")
    sw = workloads.gen_scales(8, N, "float16")
    acc, out = run(rbq, qa, sa, qw, sw)
    acc_ref = oracle.int_gemm(oracle.unpack_nibbles(qa), oracle.unpack_nibbles(qw))
    check_out(acc, out, acc_ref, sa, sw)


@pytest.mark.parametrize("M,N,K", SMALL_M)
def test_w4a8_few_tokens(rbq, M, N, K):
    print(f"case w4a8_gemm few tokens M={M} N={N} K={K}", flush=True)
    qa = gen_int8_codes(5, M, K)
    qw = workloads.gen_packed_codes(6, N, K)
    sa = workloads.gen_scales(7, M, "float32")
    sw = workloads.gen_scales(8, N, "float32")
    acc, out = run8(rbq, qa, sa, qw, sw)
    acc_ref, _ = oracle.w4a8_gemm(qa, sa, oracle.unpack_nibbles(qw), sw)
    check_out(acc, out, acc_ref, sa, sw)


@pytest.mark.parametrize("which", ["w4a4", "w4a8"])
def test_few_token_kernel_matches_tiled_kernel(rbq, which):
    """64 tokens go to the few-token kernel, 65 to the tiled one: on the same first 64
    tokens both give the same int32 sums and, with the same epilogue arithmetic, the same
    bf16 bits."""
    N, K = 1032, 2048
    print(f"case {which} few-token vs tiled", flush=True)
    qa = workloads.gen_packed_codes(9, 65, K) if which == "w4a4" else gen_int8_codes(9, 65, K)
    qw = dev(workloads.gen_packed_codes(10, N, K))
    sa = dev(workloads.gen_scales(11, 65, "float16"))
    sw = dev(workloads.gen_scales(12, N, "float16"))
    call = rbq.w4a4_gemm if which == "w4a4" else rbq.w4a8_gemm
    big_out, big_acc = call(dev(qa), sa, qw, sw, return_acc=True)
    small_out, small_acc = call(dev(qa[:64]), sa[:64].contiguous(), qw, sw, return_acc=True)
    torch.cuda.synchronize()
    assert torch.equal(small_acc, big_acc[:64])
    assert torch.equal(small_out.view(torch.int16), big_out[:64].view(torch.int16))
