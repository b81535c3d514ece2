"""GPU parity of the group-wise scale variants against the fp64 oracle, through the C ABI:
quantize_groups_int4 (one absmax scale per run of G elements of rows already in the
rotated basis) and w4a8_gemm_grouped (INT8 activations x packed INT4 weights with
group-wise weight scales): scales exact in the stored dtype, codes bit-exact (the
quantizer's rounding decision is exact), GEMM outputs within 1e-2 relative of the exact
product plus the fp32 accumulation bound of the scaled group sums (``check_grouped``)."""

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


def to_dev(x, dtype):
    if dtype == "float32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
        t = t.view(torch.bfloat16 if dtype == "bfloat16" else torch.float16)
    return t.cuda()


@pytest.mark.parametrize("group", [32, 64, 128, 256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "float16"])
def test_quantize_groups(rbq, group, dtype):
    K, rows = 8192, 37
    print(f"case quantize_groups_int4 group={group} dtype={dtype}", flush=True)
    y = workloads.gen_rows(group, rows, K, dtype, n_outliers=3, factor=30)
    codes, scales = rbq.quantize_groups_int4(to_dev(y, dtype), group)
    torch.cuda.synchronize()
    ref = oracle.quantize_groups(workloads.to_float64(y, dtype), group, "float16", packed=True)
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), ref["s_stored"])
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])


def test_quantize_groups_unpacked_fp32_scales_strided_and_ragged(rbq):
    K, rows, group = 4096, 1001, 256
    print("case quantize_groups_int4 unpacked fp32 scales strided", flush=True)
    y = workloads.gen_rows(5, rows, K + 32, "float32", n_outliers=1, factor=50)
    y[7, :] = 0.0                                                     # an all-zero row
    yd = to_dev(y, "float32")[:, :K]
    codes, scales = rbq.quantize_groups_int4(yd, group, packed=False, scale_dtype=torch.float32)
    ref = oracle.quantize_groups(y[:, :K].astype(np.float64), group, "float32", packed=False)
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), ref["s_stored"])
    assert np.array_equal(codes.cpu().numpy().view(np.int8), ref["q"])


def check_grouped(out_dev, partial, out_ref, sa, sw):
    """bf16 outputs against the exact product: |got - ref| <= 1e-2 |ref| + (G + 2) 2^-24 T,
    where G = K / group and T = |sa| sum_g |sw[n, g] partial_g|: the group sums are exact
    integers, and the fp32 steps (G products with the group scale, G additions, the product
    with sa) each round by at most 2^-24 relative to a value bounded by T; the final bf16
    rounding is within the relative term. Outputs whose every group sum is 0 must be 0."""
    got = out_dev.float().cpu().numpy().astype(np.float64)
    sa = np.asarray(sa, dtype=np.float64)
    sw = np.asarray(sw, dtype=np.float64)
    terms = np.zeros_like(out_ref)
    for g in range(partial.shape[0]):
        terms += np.abs(partial[g].astype(np.float64) * sw[None, :, g])
    terms *= np.abs(sa)[:, None]
    zero = terms == 0
    assert np.all(got[zero] == 0)
    err = np.abs(got - out_ref)
    bound = 1e-2 * np.abs(out_ref) + (partial.shape[0] + 2) * 2.0 ** -24 * terms
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    assert np.all(err <= bound), f"worst error {worst:.3g}x the bound"


def _weights_and_activations(seed, M, N, K, group):
    """A: bf16 rows -> INT8 codes per token; W: fp32 rows -> INT4 codes per group; both
    rotated first when K is a power of two and quantized by the oracle (operands identical
    on both sides; the product does not depend on how the codes were made)."""
    rot = K & (K - 1) == 0
    a = workloads.gen_rows(seed, M, K, "bfloat16", n_outliers=1, factor=40)
    w = workloads.gen_rows(seed + 1, N, K, "float32", n_outliers=0) * np.float32(0.02)
    w64 = oracle.rotate(w.astype(np.float64)) if rot else w.astype(np.float64)
    rw = oracle.quantize_groups(w64, group, "float16", packed=True)
    ra = oracle.hadamard_quant_int4(workloads.to_float64(a, "bfloat16"), "float16", packed=False, bits=8,
                                    rotate_input=rot)
    return ra, rw


@pytest.mark.parametrize("M,N,K,group", [(1, 8, 128, 128), (64, 256, 1024, 128), (300, 264, 2048, 256),
                                         (513, 1032, 4096, 256), (130, 136, 4096, 1024), (64, 64, 4096, 4096),
                                         (1, 8, 128, 32), (96, 520, 1024, 32), (257, 264, 2048, 64),
                                         (200, 1024, 4096, 32)])
def test_w4a8_gemm_grouped(rbq, M, N, K, group):
    print(f"case w4a8_gemm_grouped M={M} N={N} K={K} group={group}", flush=True)
    ra, rw = _weights_and_activations(M + N, M, N, K, group)
    out = rbq.w4a8_gemm_grouped(torch.from_numpy(ra["q"].astype(np.int8)).cuda(),
                                torch.from_numpy(ra["scales"]).cuda(),
                                torch.from_numpy(rw["codes"]).cuda(),
                                torch.from_numpy(rw["scales"]).cuda(), group)
    torch.cuda.synchronize()
    partial, ref = oracle.w4a8_gemm_grouped(ra["q"], ra["s_stored"], rw["q"], rw["s_stored"], group)
    check_grouped(out, partial, ref, ra["s_stored"], rw["s_stored"])


@pytest.mark.parametrize("group", [256, 64, 32])
def test_w4a8_gemm_grouped_random_codes_extremes(rbq, group):
    # uniform random codes over the full grids and log-uniform scales, including -128 / -8
    M, N, K = 256, 512, 4096
    print(f"case w4a8_gemm_grouped random codes group={group}", flush=True)
    rng = np.random.default_rng(12)
    qa = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    qw = workloads.gen_packed_codes(13, N, K)
    sa = workloads.gen_scales(14, M, "float32")
    sw = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(N, K // group))).astype(np.float32)
    out = rbq.w4a8_gemm_grouped(torch.from_numpy(qa).cuda(), torch.from_numpy(sa).cuda(),
                                torch.from_numpy(qw).cuda(), torch.from_numpy(sw).cuda(), group)
    partial, ref = oracle.w4a8_gemm_grouped(qa, sa, oracle.unpack_nibbles(qw), sw, group)
    check_grouped(out, partial, ref, sa, sw)


@pytest.mark.parametrize("group", [256, 32])
def test_w4a8_gemm_grouped_full_size_sampled(rbq, group):
    """4096 x 11008 x 4096 with groups of 256 and of 32: rows sampled against the oracle,
    and two calls bit-identical."""
    M, N, K = 4096, 11008, 4096
    print(f"case w4a8_gemm_grouped full size group={group}", flush=True)
    rng = np.random.default_rng(21)
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = workloads.gen_packed_codes(22, N, K)
    sa = workloads.gen_scales(23, M, "float16")
    sw = workloads.gen_scales(24, N * (K // group), "float16").reshape(N, K // group)
    args = (torch.from_numpy(qa).cuda(), torch.from_numpy(sa).cuda(), torch.from_numpy(qw).cuda(),
            torch.from_numpy(sw).cuda(), group)
    out = rbq.w4a8_gemm_grouped(*args)
    out2 = rbq.w4a8_gemm_grouped(*args)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    rows = np.unique(np.concatenate([[0, 1, 4095], rng.integers(0, M, 13)]))
    partial, ref = oracle.w4a8_gemm_grouped(qa[rows], sa[rows], oracle.unpack_nibbles(qw), sw, group)
    check_grouped(out[torch.from_numpy(rows).cuda()], partial, ref, sa[rows], sw)


@pytest.mark.parametrize("group", [32, 4096])
def test_w4a8_gemm_grouped_largest_k_extremes(rbq, group):
    """K = 65536 with every code at its extreme (-128 x -8): each group sum is 1024 x group,
    up to 2048 groups per output; random scales."""
    M, N, K = 32, 64, 65536
    print(f"case w4a8_gemm_grouped K=65536 extremes group={group}", flush=True)
    rng = np.random.default_rng(77 + group)
    qa = np.full((M, K), -128, dtype=np.int8)
    qw = np.full((N, K // 2), 0x88, dtype=np.uint8)  # -8 in both nibbles
    sa = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), M)).astype(np.float32)
    sw = np.exp(rng.uniform(np.log(1e-4), np.log(1e-2), (N, K // group))).astype(np.float32)
    out = rbq.w4a8_gemm_grouped(torch.from_numpy(qa).cuda(), torch.from_numpy(sa).cuda(),
                                torch.from_numpy(qw).cuda(), torch.from_numpy(sw).cuda(), group)
    partial, ref = oracle.w4a8_gemm_grouped(qa, sa, oracle.unpack_nibbles(qw), sw, group)
    assert np.all(partial == 1024 * group)
    check_grouped(out, partial, ref, sa, sw)


# Few tokens (M <= 64, decode): the grouped product on the kernel where each wave takes a
# contiguous range of K, folds at group and range ends, and the waves add their fp32 sums at
# the end; every group size class, ragged N, ranges that cut groups (K = 11008 and a group
# of all K), and waves with no steps (K = 128).
@pytest.mark.parametrize("M,N,K,group", [(16, 11008, 4096, 256), (16, 520, 4096, 32), (33, 264, 2048, 64),
                                         (5, 136, 1024, 1024), (64, 1032, 4096, 128), (1, 8, 4096, 32),
                                         (3, 264, 11008, 256), (7, 72, 11008, 32), (2, 40, 4096, 4096),
                                         (9, 16, 128, 64), (40, 24, 128, 32)])
def test_w4a8_gemm_grouped_few_tokens(rbq, M, N, K, group):
    print(f"case w4a8_gemm_grouped few tokens M={M} N={N} K={K} group={group}", flush=True)
    ra, rw = _weights_and_activations(M + N + K, M, N, K, group)
    out = rbq.w4a8_gemm_grouped(torch.from_numpy(ra["q"].astype(np.int8)).cuda(),
                                torch.from_numpy(ra["scales"]).cuda(),
                                torch.from_numpy(rw["codes"]).cuda(),
                                torch.from_numpy(rw["scales"]).cuda(), group)
    torch.cuda.synchronize()
    partial, ref = oracle.w4a8_gemm_grouped(ra["q"], ra["s_stored"], rw["q"], rw["s_stored"], group)
    check_grouped(out, partial, ref, ra["s_stored"], rw["s_stored"])


@pytest.mark.parametrize("M,group", [(7, 256), (40, 32), (1, 64)])
def test_w4a8_gemm_grouped_few_tokens_fp32_scales_random_codes(rbq, M, group):
    # the few-token kernel with fp32 scales, codes over the full grids (-128 / -8 included)
    N, K = 264, 2048
    print(f"case w4a8_gemm_grouped few tokens fp32 scales M={M} group={group}", flush=True)
    rng = np.random.default_rng(31 + M)
    qa = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    qw = workloads.gen_packed_codes(32 + M, N, K)
    sa = workloads.gen_scales(33 + M, M, "float32")
    sw = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(N, K // group))).astype(np.float32)
    out = rbq.w4a8_gemm_grouped(torch.from_numpy(qa).cuda(), torch.from_numpy(sa).cuda(),
                                torch.from_numpy(qw).cuda(), torch.from_numpy(sw).cuda(), group)
    partial, ref = oracle.w4a8_gemm_grouped(qa, sa, oracle.unpack_nibbles(qw), sw, group)
    check_grouped(out, partial, ref, sa, sw)
