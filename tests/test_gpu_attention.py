"""GPU parity of attention_decode_int4kv and attention_decode_int4kv_split against the fp64
oracle, through the C ABI: the kernels and the oracle read the same INT4 key/value codes and
scales.

Tolerance, derived from the kernel's fp32 arithmetic: a score takes the rounded product of
the query with the softmax scale, 32 fused multiply-adds per lane, 2 shuffle additions
across the four lanes of a token and one product with the key scale, so its error is at most
d_s = 36 * 2^-24 * |scale| * k_scale[s] * sum_d |q_d code_sd|; the probabilities then err by
at most 2 max(d_s) + 2^-20 relative (each is a product of at most S/256 + 3 exponentials:
the token's own, its group's rescalings and the merge weights (one more for the split
kernel's ranges), whose arguments add up to the score's distance from the maximum), the sums
over S tokens by S * 2^-23,
the output is rounded to bf16 (2^-8 relative covers it) or fp16 (2^-8 relative, plus
2^-25 absolute: half the spacing of fp16's subnormals, which is all the precision left to
an output below 2^-14, as in a peaked softmax whose winning value is 0 in some dim), and
probabilities below the fp32 normal range (2^-126) are flushed to zero:
    |out - ref| <= 2^-8 |ref| + (2 max_s d_s + 2^-20 + S 2^-23) * sum_s p_s |v_sd|
                   + S 2^-126 max_s |v_sd|  (+ 2^-25 for fp16 outputs)."""

import math

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


def bf16(x):
    return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def check(out_dev, q, kc, ks, vc, vs, scale, heads=None):
    """heads: optional list of (b, h) to check (the oracle then runs on those only)."""
    floor = 2.0 ** -25 if out_dev.dtype == torch.float16 else 0.0
    got = out_dev.float().cpu().numpy().astype(np.float64)
    B, H, D = q.shape
    Hkv = kc.shape[1]
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        kvh = h // (H // Hkv)
        sl = (slice(b, b + 1), slice(kvh, kvh + 1))
        ref, p = oracle.attention_decode(q[b:b + 1, h:h + 1], kc[sl], ks[sl], vc[sl], vs[sl], scale)
        ref, p = ref[0, 0], p[0, 0]
        S = p.shape[0]
        dots = np.abs(kc[b, kvh].astype(np.float64) * q[b, h][None, :]).sum(axis=1)
        d_max = float(np.max(36 * 2.0 ** -24 * abs(scale) * ks[b, kvh].astype(np.float64) * dots))
        vmag = (p[:, None] * np.abs(vc[b, kvh] * vs[b, kvh][:, None].astype(np.float64))).sum(axis=0)
        vmax = float(np.max(np.abs(vc[b, kvh] * vs[b, kvh][:, None].astype(np.float64))))
        bound = (2.0 ** -8 * np.abs(ref) + (2 * d_max + 2.0 ** -20 + S * 2.0 ** -23) * vmag
                 + S * 2.0 ** -126 * vmax + floor)
        err = np.abs(got[b, h] - ref)
        assert np.all(err <= bound), f"(b={b}, h={h}) worst {float(np.max(err / np.maximum(bound, 1e-300))):.3g}x bound"


def make(seed, B, H, Hkv, S, cap, scale_dtype=np.float16):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((B, H, 128)))
    kc = rng.integers(-8, 8, size=(B, Hkv, cap, 128)).astype(np.int8)
    vc = rng.integers(-8, 8, size=(B, Hkv, cap, 128)).astype(np.int8)
    ks = np.exp(rng.uniform(np.log(0.02), np.log(0.5), size=(B, Hkv, cap))).astype(scale_dtype)
    vs = np.exp(rng.uniform(np.log(0.02), np.log(0.5), size=(B, Hkv, cap))).astype(scale_dtype)
    return q, kc, ks, vc, vs


def run(rbq, q, kc, ks, vc, vs, scale, seq, splits=None):
    """splits: None for attention_decode_int4kv, else attention_decode_int4kv_split."""
    qd = torch.from_numpy(workloads.f32_to_bf16_bits(q.astype(np.float32)).view(np.int16)).view(torch.bfloat16).cuda()
    pk = lambda c: torch.from_numpy(oracle.pack_nibbles(c.reshape(-1, 128)).reshape(c.shape[:-1] + (64,))).cuda()
    args = (qd, pk(kc), torch.from_numpy(ks).cuda(), pk(vc), torch.from_numpy(vs).cuda(), scale)
    if splits is None:
        out = rbq.attention_decode_int4kv(*args, seq=seq)
    else:
        out = rbq.attention_decode_int4kv_split(*args, splits, seq=seq)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("B,H,Hkv,S,cap", [(1, 1, 1, 1, 1), (2, 4, 2, 37, 40), (1, 8, 8, 1024, 1024),
                                           (2, 32, 8, 3000, 3072), (3, 6, 3, 1025, 1100)])
def test_attention_random_codes(rbq, B, H, Hkv, S, cap):
    print(f"case attention B={B} H={H} Hkv={Hkv} S={S} cap={cap}", flush=True)
    q, kc, ks, vc, vs = make(B * 100 + S, B, H, Hkv, S, cap)
    scale = 1.0 / math.sqrt(128)
    out = run(rbq, q, kc, ks, vc, vs, scale, S)
    check(out, q, kc[:, :, :S], ks[:, :, :S], vc[:, :, :S], vs[:, :, :S], scale)


def test_attention_fp32_scales_and_peaked_scores(rbq):
    # a large scale makes the softmax nearly one-hot: the running maximum must be exact
    q, kc, ks, vc, vs = make(7, 2, 4, 4, 2500, 2500, np.float32)
    out = run(rbq, q, kc, ks, vc, vs, 4.0, 2500)
    check(out, q, kc, ks, vc, vs, 4.0)


def test_attention_fp16_query_and_output(rbq):
    # the query (and so the output) in fp16; the bound's 2^-8 output term covers fp16 rounding
    B, H, Hkv, S, cap = 2, 8, 4, 700, 768
    print("case attention fp16 query", flush=True)
    _, kc, ks, vc, vs = make(41, B, H, Hkv, S, cap)
    q = np.random.default_rng(42).standard_normal((B, H, 128)).astype(np.float16).astype(np.float64)
    pk = lambda c: torch.from_numpy(oracle.pack_nibbles(c.reshape(-1, 128)).reshape(c.shape[:-1] + (64,))).cuda()
    qd = torch.from_numpy(q.astype(np.float16)).cuda()
    scale = 1.0 / math.sqrt(128)
    out = rbq.attention_decode_int4kv(qd, pk(kc), torch.from_numpy(ks).cuda(), pk(vc), torch.from_numpy(vs).cuda(),
                                      scale, seq=S)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    check(out, q, kc[:, :, :S], ks[:, :, :S], vc[:, :, :S], vs[:, :, :S], scale)


def test_attention_end_to_end_with_the_kv_cache_writers(rbq):
    """Q and K through kv_rotate_quant (Q rotated only, K rotated and quantized), V through
    hadamard_quant_int4 without rotation: the kernel reads exactly what the writers wrote,
    and its output is close to full-precision attention on the unquantized inputs."""
    B, H, S, D = 2, 4, 512, 128
    # no outlier channels here: with them the scores are so peaked that the sanity bound on
    # the deviation from unquantized attention (last assertion) would not be meaningful
    q_bits, k_bits, _ = workloads.gen_kv(seed=5, batch=B, heads=H, seq=S, head_dim=D, n_outliers=0)
    v_bits = workloads.gen_rows(6, B * H * S, D, "bfloat16", n_outliers=0).reshape(B, H, S, D)
    q_last = q_bits[:, :, -1:, :]                                  # the decode query: last position
    to = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    # the query rotated (not quantized); the keys of every position rotated and quantized
    r = rbq.kv_rotate_quant(to(q_last), to(q_last), q_rotate_only=True)
    r2 = rbq.kv_rotate_quant(to(k_bits), to(k_bits))
    kc, ks = r2["k_codes"], r2["k_scales"]
    vcodes, vscales = rbq.hadamard_quant_int4(to(v_bits.reshape(-1, D)), rotate=False)
    q_rot = r["q_rotated"].reshape(B, H, D).contiguous()
    scale = 1.0 / math.sqrt(D)
    out = rbq.attention_decode_int4kv(q_rot, kc, ks, vcodes.reshape(B, H, S, D // 2), vscales.reshape(B, H, S), scale)
    torch.cuda.synchronize()
    q_np = q_rot.float().cpu().numpy().astype(np.float64)
    kq = oracle.unpack_nibbles(kc.cpu().numpy().reshape(-1, D // 2)).reshape(B, H, S, D)
    vq = oracle.unpack_nibbles(vcodes.cpu().numpy()).reshape(B, H, S, D)
    check(out, q_np, kq, ks.cpu().numpy(), vq, vscales.cpu().numpy().reshape(B, H, S), scale)
    # against unquantized attention (unrotated q, k): quantization error only
    full, _ = oracle.attention_decode(workloads.to_float64(q_last, "bfloat16")[:, :, 0],
                                      workloads.to_float64(k_bits, "bfloat16"), np.ones((B, H, S)),
                                      workloads.to_float64(v_bits, "bfloat16"), np.ones((B, H, S)), scale)
    got = out.float().cpu().numpy()
    rel = np.linalg.norm(got - full) / np.linalg.norm(full)
    print(f"relative deviation from unquantized attention: {rel:.4f}")
    assert rel < 0.2  # a sanity check of the chain, not parity (the codes are the parity check)


def test_attention_full_decode_shape_sampled(rbq):
    """B = 16, H = 32, S = 2048 (the R3 workload's cache), heads sampled against the oracle."""
    B, H, S = 16, 32, 2048
    print("case attention full decode shape", flush=True)
    q, kc, ks, vc, vs = make(99, B, H, H, S, S)
    out = run(rbq, q, kc, ks, vc, vs, 1.0 / math.sqrt(128), S)
    rng = np.random.default_rng(3)
    pairs = [(0, 0), (15, 31)] + [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(10)]
    check(out, q, kc, ks, vc, vs, 1.0 / math.sqrt(128), heads=pairs)


@pytest.mark.parametrize("B,H,Hkv,S,cap,splits", [(1, 1, 1, 1, 1, 1), (1, 1, 1, 1, 1, 5), (2, 4, 2, 37, 40, 3),
                                                  (2, 4, 2, 37, 40, 64), (1, 8, 8, 1024, 1024, 4),
                                                  (2, 32, 8, 3000, 3072, 7), (3, 6, 3, 1025, 1100, 16)])
def test_attention_split_random_codes(rbq, B, H, Hkv, S, cap, splits):
    """ranges of ceil(S / splits) tokens; with splits > S the last ranges are empty"""
    print(f"case attention split B={B} H={H} Hkv={Hkv} S={S} cap={cap} splits={splits}", flush=True)
    q, kc, ks, vc, vs = make(B * 100 + S, B, H, Hkv, S, cap)
    scale = 1.0 / math.sqrt(128)
    out = run(rbq, q, kc, ks, vc, vs, scale, S, splits=splits)
    check(out, q, kc[:, :, :S], ks[:, :, :S], vc[:, :, :S], vs[:, :, :S], scale)


def test_attention_split_peaked_scores_fp32_scales(rbq):
    # nearly one-hot softmax: the ranges' maxima differ widely and all but one weigh ~0
    print("case attention split peaked", flush=True)
    q, kc, ks, vc, vs = make(7, 2, 4, 4, 2500, 2500, np.float32)
    out = run(rbq, q, kc, ks, vc, vs, 4.0, 2500, splits=9)
    check(out, q, kc, ks, vc, vs, 4.0)


def test_attention_split_full_decode_shape_sampled(rbq):
    """B = 16, H = 32, S = 2048 with 8 ranges per head, in a reused workspace; heads sampled
    against the oracle, and the whole output within a few bf16 steps of the unsplit kernel's."""
    B, H, S = 16, 32, 2048
    print("case attention split full decode shape", flush=True)
    q, kc, ks, vc, vs = make(99, B, H, H, S, S)
    scale = 1.0 / math.sqrt(128)
    ws = torch.full((rbq.attention_split_workspace_bytes(B, H, 8),), 0xFF, dtype=torch.uint8, device="cuda")
    qd = torch.from_numpy(workloads.f32_to_bf16_bits(q.astype(np.float32)).view(np.int16)).view(torch.bfloat16).cuda()
    pk = lambda c: torch.from_numpy(oracle.pack_nibbles(c.reshape(-1, 128)).reshape(c.shape[:-1] + (64,))).cuda()
    args = (qd, pk(kc), torch.from_numpy(ks).cuda(), pk(vc), torch.from_numpy(vs).cuda(), scale)
    out = rbq.attention_decode_int4kv_split(*args, 8, workspace=ws)
    out2 = rbq.attention_decode_int4kv_split(*args, 8, workspace=ws)  # the workspace as the first call left it
    ref = rbq.attention_decode_int4kv(*args)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    rng = np.random.default_rng(3)
    pairs = [(0, 0), (15, 31)] + [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(10)]
    check(out, q, kc, ks, vc, vs, scale, heads=pairs)
    # the two kernels' fp32 values differ by rounding only, so their bf16 outputs by at most
    # about one bf16 step (2^-7 relative); 2^-6 leaves room for a binade edge
    a, b = out.float(), ref.float()
    assert bool(((a - b).abs() <= b.abs() * 2.0 ** -6 + 2.0 ** -20).all())


# Grouped key/value heads with enough (batch, key/value head[, range]) triples for the
# shared-load kernel (one workgroup per set of 2 or 4 query heads loads each cached token
# once for all of them): 2, 4 and 8 query heads per key/value head, ragged lengths.
@pytest.mark.parametrize("B,H,Hkv,S,cap", [(32, 32, 8, 300, 320), (16, 32, 16, 129, 129), (16, 64, 8, 257, 300),
                                           (32, 24, 4, 513, 520)])
def test_attention_grouped_heads_shared_loads(rbq, B, H, Hkv, S, cap):
    print(f"case attention shared B={B} H={H} Hkv={Hkv} S={S} cap={cap}", flush=True)
    q, kc, ks, vc, vs = make(B * 7 + H + S, B, H, Hkv, S, cap)
    scale = 1.0 / math.sqrt(128)
    out = run(rbq, q, kc, ks, vc, vs, scale, S)
    rng = np.random.default_rng(S)
    pairs = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(40)]
    check(out, q, kc[:, :, :S], ks[:, :, :S], vc[:, :, :S], vs[:, :, :S], scale, heads=pairs)


@pytest.mark.parametrize("B,H,Hkv,S,cap,splits", [(4, 32, 8, 2000, 2048, 8), (4, 32, 8, 5, 8, 8),
                                                  (8, 16, 8, 777, 800, 16)])
def test_attention_split_grouped_heads_shared_loads(rbq, B, H, Hkv, S, cap, splits):
    """the split form over the shared-load kernel, including ranges past the sequence's end"""
    print(f"case attention split shared B={B} H={H} Hkv={Hkv} S={S} cap={cap} splits={splits}", flush=True)
    q, kc, ks, vc, vs = make(B * 11 + S, B, H, Hkv, S, cap)
    scale = 1.0 / math.sqrt(128)
    out = run(rbq, q, kc, ks, vc, vs, scale, S, splits=splits)
    check(out, q, kc[:, :, :S], ks[:, :, :S], vc[:, :, :S], vs[:, :, :S], scale)


def test_attention_shared_loads_fp32_scales_peaked_fp16_query(rbq):
    # nearly one-hot softmax, fp32 scales and an fp16 query through the shared-load kernel
    B, H, Hkv, S = 32, 32, 8, 600
    print("case attention shared peaked fp16", flush=True)
    _, kc, ks, vc, vs = make(43, B, H, Hkv, S, S, np.float32)
    q = np.random.default_rng(44).standard_normal((B, H, 128)).astype(np.float16).astype(np.float64)
    pk = lambda c: torch.from_numpy(oracle.pack_nibbles(c.reshape(-1, 128)).reshape(c.shape[:-1] + (64,))).cuda()
    qd = torch.from_numpy(q.astype(np.float16)).cuda()
    out = rbq.attention_decode_int4kv(qd, pk(kc), torch.from_numpy(ks).cuda(), pk(vc), torch.from_numpy(vs).cuda(), 4.0)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    rng = np.random.default_rng(45)
    pairs = [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(40)]
    check(out, q, kc, ks, vc, vs, 4.0, heads=pairs)
