"""GPU parity of kv_cache_append_int4 against the fp64 oracle, through the C ABI: RoPE ->
R3 -> INT4 keys and INT4 values appended at position pos0 of a cache whose capacity is
larger than the tokens written, queries RoPE'd and rotated in 16 bits; and the chain
RoPE -> R3 -> append -> attention_decode_int4kv over the cache the appends wrote.

Keys: the oracle's RoPE is the exact map rounded once to the 16-bit format, with either
neighbour accepted where float32 evaluation error reaches a rounding midpoint
(tests/parity.py); values: quantized as they are, codes exact; cache rows outside the
written positions keep their sentinel bytes."""

import math

import numpy as np
import pytest

import oracle
import workloads
from parity import check_quant, check_rope_quant, check_rope_rotated

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 0xA5


@pytest.fixture(scope="module")
def rbq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_bit_quantization_fwht_amd as m

    m.lib()
    return m


def rope_tables(positions, d, base=10000.0):
    inv = base ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)
    th = np.outer(np.arange(positions, dtype=np.float64), inv)
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


def bhsd_view(bits, dtype):
    """[B, H, S, D] 16-bit values laid out in memory as [B, S, H, D] (a strided view)."""
    t = torch.from_numpy(np.ascontiguousarray(bits.transpose(0, 2, 1, 3)).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == "bfloat16" else torch.float16).cuda()
    return t.permute(0, 2, 1, 3)


def gen(seed, B, H, S, D, dtype):
    q, k, _ = workloads.gen_kv(seed=seed, batch=B, heads=H, seq=S, head_dim=D)
    if dtype == "float16":
        q = workloads.bf16_bits_to_f32(q).astype(np.float16).view(np.uint16)
        k = workloads.bf16_bits_to_f32(k).astype(np.float16).view(np.uint16)
    return q, k


def empty_cache(B, Hkv, cap, D, sdt=torch.float16):
    kc = torch.full((B, Hkv, cap, D // 2), SENTINEL, dtype=torch.uint8, device="cuda")
    vc = torch.full((B, Hkv, cap, D // 2), SENTINEL, dtype=torch.uint8, device="cuda")
    ks = torch.full((B, Hkv, cap), -7.0, dtype=sdt, device="cuda")
    vs = torch.full((B, Hkv, cap), -7.0, dtype=sdt, device="cuda")
    return kc, ks, vc, vs


def check_rows(rbq_out, x_bits, dtype, pos0, tables, rotate, sdt="float16"):
    """rbq_out = (codes [B, Hkv, cap, D/2], scales [B, Hkv, cap]) after one append of
    x_bits [B, Hkv, S, D] at pos0; tables = (cos, sin) or None."""
    codes, scales = (t.cpu().numpy() for t in rbq_out)
    B, Hkv, S, D = x_bits.shape
    rows = B * Hkv * S
    got_q = oracle.unpack_nibbles(codes[:, :, pos0:pos0 + S].reshape(rows, D // 2))
    got_s = scales[:, :, pos0:pos0 + S].reshape(rows).astype(np.float64)
    x = workloads.to_float64(x_bits, dtype).reshape(rows, D)
    if tables is not None:
        cos, sin = tables
        pos = pos0 + np.arange(S)
        cr = np.broadcast_to(cos[pos][None, None], (B, Hkv, S, D // 2)).reshape(rows, D // 2)
        sr = np.broadcast_to(sin[pos][None, None], (B, Hkv, S, D // 2)).reshape(rows, D // 2)
        return check_rope_quant(got_q, got_s, x, cr, sr, dtype, scale_dtype=sdt)
    ref = oracle.hadamard_quant_int4(x, sdt, packed=False, rotate_input=rotate)
    st = check_quant(got_q, got_s, ref, sdt, x, rotate=rotate)
    if not rotate:
        assert st["code_flips"] == 0
    return st


def assert_untouched(t, pos0, S, sentinel):
    a = t.cpu().numpy()
    outside = np.ones(a.shape[2], dtype=bool)
    outside[pos0:pos0 + S] = False
    assert np.all(a[:, :, outside] == sentinel)


@pytest.mark.parametrize("shape", [(2, 6, 3, 37, 96, 29), (2, 8, 4, 32, 80, 16)])
@pytest.mark.parametrize("rope", [True, False])
@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_append_into_cache(rbq, D, dtype, rope, shape):
    """shape = (B, H, Hkv, S, cap, pos0); the second takes the RoPE kernels' head-group
    order for Q (and for K at head_dim 128)."""
    B, H, Hkv, S, cap, pos0 = shape
    print(f"case kv_cache_append D={D} {dtype} rope={rope} shape={shape}", flush=True)
    q_bits, _ = gen(D + 1, B, H, S, D, dtype)
    k_bits, v_bits = gen(D + 2, B, Hkv, S, D, dtype)
    q, k, v = bhsd_view(q_bits, dtype), bhsd_view(k_bits, dtype), bhsd_view(v_bits, dtype)
    cos, sin = rope_tables(pos0 + S + 5, D)
    kc, ks, vc, vs = empty_cache(B, Hkv, cap, D)
    kw = {"rope_cos": torch.from_numpy(cos).cuda(), "rope_sin": torch.from_numpy(sin).cuda()} if rope else {}
    qr = rbq.kv_cache_append_int4(k, v, kc, ks, vc, vs, pos0, q=q, **kw)
    torch.cuda.synchronize()
    for t in (kc, vc):
        assert_untouched(t, pos0, S, SENTINEL)
    for t in (ks, vs):
        assert_untouched(t.float(), pos0, S, -7.0)
    tables = (cos, sin) if rope else None
    print("  k:", check_rows((kc, ks), k_bits, dtype, pos0, tables, True), flush=True)
    print("  v:", check_rows((vc, vs), v_bits, dtype, pos0, None, False), flush=True)
    got = qr.float().cpu().numpy().astype(np.float64).reshape(B * H * S, D)
    x = workloads.to_float64(q_bits, dtype).reshape(B * H * S, D)
    if rope:
        pos = pos0 + np.arange(S)
        cr = np.broadcast_to(cos[pos][None, None], (B, H, S, D // 2)).reshape(-1, D // 2)
        sr = np.broadcast_to(sin[pos][None, None], (B, H, S, D // 2)).reshape(-1, D // 2)
        check_rope_rotated(got, x, cr, sr, dtype)
    else:
        want = oracle.round_to_format(oracle.rotate(x), dtype)
        step = 2.0 ** -7 if dtype == "bfloat16" else 2.0 ** -10
        assert np.all(np.abs(got - want) <= np.abs(want) * step + 2.0 ** -24)
        assert np.mean(got == want) > 0.999


def test_append_fp32_scales_no_query_and_errors(rbq):
    B, Hkv, S, D, cap, pos0 = 1, 4, 9, 128, 16, 7
    print("case kv_cache_append fp32 scales, no query", flush=True)
    k_bits, v_bits = gen(77, B, Hkv, S, D, "bfloat16")
    k, v = bhsd_view(k_bits, "bfloat16"), bhsd_view(v_bits, "bfloat16")
    kc, ks, vc, vs = empty_cache(B, Hkv, cap, D, sdt=torch.float32)
    assert rbq.kv_cache_append_int4(k, v, kc, ks, vc, vs, pos0) is None
    torch.cuda.synchronize()
    check_rows((kc, ks), k_bits, "bfloat16", pos0, None, True, sdt="float32")
    check_rows((vc, vs), v_bits, "bfloat16", pos0, None, False, sdt="float32")
    assert_untouched(kc, pos0, S, SENTINEL)
    with pytest.raises(rbq.RBQError):  # pos0 + S beyond the capacity
        rbq.kv_cache_append_int4(k, v, kc, ks, vc, vs, cap - S + 1)
    k32 = torch.zeros((1, 2, 3, 32), dtype=torch.bfloat16, device="cuda")
    c32 = torch.zeros((1, 2, 8, 16), dtype=torch.uint8, device="cuda")
    s32 = torch.zeros((1, 2, 8), dtype=torch.float16, device="cuda")
    with pytest.raises(rbq.RBQError) as e:  # head_dim 32 has no cache kernel
        rbq.kv_cache_append_int4(k32, k32.clone(), c32, s32, c32.clone(), s32.clone(), 0)
    assert e.value.status == rbq.RBQ_ENOTSUP


def test_prefill_then_decode_chain_to_attention(rbq):
    """RoPE -> R3 -> KV4 append for a prefill of 100 tokens, then one decode token at
    position 100, then decode attention of that token's query over the 101 cached tokens.
    Each stage is checked against the oracle; the attention output against the oracle's
    attention over the cache the appends wrote, with the query the append returned."""
    B, H, Hkv, D, S1, cap = 2, 8, 2, 128, 100, 160
    print("case kv cache chain: prefill 100 + decode 1 -> attention", flush=True)
    cos, sin = rope_tables(cap, D)
    cd, sd = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    kc, ks, vc, vs = empty_cache(B, Hkv, cap, D)
    k1, v1 = gen(5, B, Hkv, S1, D, "bfloat16")
    rbq.kv_cache_append_int4(bhsd_view(k1, "bfloat16"), bhsd_view(v1, "bfloat16"), kc, ks, vc, vs, 0,
                             rope_cos=cd, rope_sin=sd)
    q2, _ = gen(6, B, H, 1, D, "bfloat16")
    k2, v2 = gen(7, B, Hkv, 1, D, "bfloat16")
    qr = rbq.kv_cache_append_int4(bhsd_view(k2, "bfloat16"), bhsd_view(v2, "bfloat16"), kc, ks, vc, vs, S1,
                                  q=bhsd_view(q2, "bfloat16"), rope_cos=cd, rope_sin=sd)
    out = rbq.attention_decode_int4kv(qr[:, :, 0, :].contiguous(), kc, ks, vc, vs, 1.0 / math.sqrt(D), seq=S1 + 1)
    torch.cuda.synchronize()
    check_rows((kc, ks), k1, "bfloat16", 0, (cos, sin), True)
    check_rows((kc, ks), k2, "bfloat16", S1, (cos, sin), True)
    check_rows((vc, vs), v1, "bfloat16", 0, None, False)
    check_rows((vc, vs), v2, "bfloat16", S1, None, False)
    assert_untouched(kc, 0, S1 + 1, SENTINEL)
    x = workloads.to_float64(q2, "bfloat16").reshape(B * H, D)
    got_q = qr.float().cpu().numpy().astype(np.float64).reshape(B * H, D)
    cr = np.broadcast_to(cos[S1], (B * H, D // 2))
    sr = np.broadcast_to(sin[S1], (B * H, D // 2))
    check_rope_rotated(got_q, x, cr, sr, "bfloat16")
    # attention: the oracle over the codes and scales the appends wrote, with the query the
    # append returned (both checked above); tolerance as in test_gpu_attention
    from test_gpu_attention import check as check_attention
    n = S1 + 1
    kcode = oracle.unpack_nibbles(kc.cpu().numpy()[:, :, :n].reshape(-1, D // 2)).reshape(B, Hkv, n, D)
    vcode = oracle.unpack_nibbles(vc.cpu().numpy()[:, :, :n].reshape(-1, D // 2)).reshape(B, Hkv, n, D)
    check_attention(out, got_q.reshape(B, H, D), kcode, ks.cpu().numpy()[:, :, :n], vcode, vs.cpu().numpy()[:, :, :n],
                    1.0 / math.sqrt(D))


@pytest.mark.parametrize("S,pos0", [(16, 48), (1, 63)])
def test_append_fills_the_cache_to_its_last_row(rbq, S, pos0):
    """pos0 + seq == seq_cap: the last rows of every head's cache (a prefill that fills it,
    and a one-token decode at the final position, with RoPE), rows before pos0 untouched."""
    B, H, Hkv, D, cap = 2, 8, 4, 128, 64
    print(f"case kv_cache_append to the last row S={S} pos0={pos0}", flush=True)
    q_bits, _ = gen(300 + S, B, H, S, D, "bfloat16")
    k_bits, v_bits = gen(301 + S, B, Hkv, S, D, "bfloat16")
    cos, sin = rope_tables(cap, D)
    kc, ks, vc, vs = empty_cache(B, Hkv, cap, D)
    qr = rbq.kv_cache_append_int4(bhsd_view(k_bits, "bfloat16"), bhsd_view(v_bits, "bfloat16"), kc, ks, vc, vs,
                                  pos0, q=bhsd_view(q_bits, "bfloat16"), rope_cos=torch.from_numpy(cos).cuda(),
                                  rope_sin=torch.from_numpy(sin).cuda())
    torch.cuda.synchronize()
    for t in (kc, vc):
        assert_untouched(t, pos0, S, SENTINEL)
    check_rows((kc, ks), k_bits, "bfloat16", pos0, (cos, sin), True)
    check_rows((vc, vs), v_bits, "bfloat16", pos0, None, False)
    got = qr.float().cpu().numpy().astype(np.float64).reshape(B * H * S, D)
    pos = pos0 + np.arange(S)
    cr = np.broadcast_to(cos[pos][None, None], (B, H, S, D // 2)).reshape(-1, D // 2)
    sr = np.broadcast_to(sin[pos][None, None], (B, H, S, D // 2)).reshape(-1, D // 2)
    check_rope_rotated(got, workloads.to_float64(q_bits, "bfloat16").reshape(B * H * S, D), cr, sr, "bfloat16")
