"""attention_decode_int4kv_split_noalloc (the split decode attention whose partials live in a
fixed device array of the library, for callers that cannot allocate) against
attention_decode_int4kv_split with a caller's workspace, through the C ABI: two calls in a
row, the second on a smaller problem, each bit-identical to the workspace entry point with
the same split count (the same kernels on the same inputs) and within the oracle's bound on
sampled heads; a problem whose partials exceed the array is refused before any launch."""

import ctypes
import math

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SCRATCH_BYTES = 8 << 20  # the library's fixed partials array


@pytest.fixture(scope="module")
def rbq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_bit_quantization_fwht_amd as m

    L = m.lib()
    vp, ci, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.attention_decode_int4kv_split_noalloc.argtypes = [vp, ci, vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64,
                                                        ctypes.c_float, i64, vp, vp]
    L.attention_decode_int4kv_split_noalloc.restype = ci
    return m


def operands(seed, B, H, Hkv, S, cap):
    rng = np.random.default_rng(seed)
    q32 = rng.standard_normal((B, H, 128)).astype(np.float32)
    q = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(q32)).astype(np.float64)
    kc = rng.integers(-8, 8, size=(B, Hkv, cap, 128)).astype(np.int8)
    vc = rng.integers(-8, 8, size=(B, Hkv, cap, 128)).astype(np.int8)
    ks = np.exp(rng.uniform(np.log(0.02), np.log(0.5), size=(B, Hkv, cap))).astype(np.float16)
    vs = np.exp(rng.uniform(np.log(0.02), np.log(0.5), size=(B, Hkv, cap))).astype(np.float16)
    host = (q, kc, ks, vc, vs)
    pk = lambda c: torch.from_numpy(oracle.pack_nibbles(c.reshape(-1, 128)).reshape(c.shape[:-1] + (64,))).cuda()
    qd = torch.from_numpy(workloads.f32_to_bf16_bits(q32).view(np.int16)).view(torch.bfloat16).cuda()
    dev = (qd, pk(kc), torch.from_numpy(ks).cuda(), pk(vc), torch.from_numpy(vs).cuda())
    return host, dev


def noalloc(rbq, dev, seq, splits, out):
    q, kc, ks, vc, vs = dev
    B, H, D = q.shape
    Hkv, cap = kc.shape[1], kc.shape[2]
    stream = torch.cuda.current_stream().cuda_stream
    return rbq.lib().attention_decode_int4kv_split_noalloc(
        q.data_ptr(), rbq.RBQ_BF16, kc.data_ptr(), ks.data_ptr(), vc.data_ptr(), vs.data_ptr(), rbq.RBQ_F16, B, H,
        Hkv, seq, cap, D, 1.0 / math.sqrt(D), splits, out.data_ptr(), stream)


def test_noalloc_matches_workspace_entry_point_twice(rbq):
    from test_gpu_attention import check

    scale = 1.0 / math.sqrt(128)
    # the first call fills most of the array; the second, smaller one reuses what it left
    for case, (B, H, Hkv, S, cap, splits) in enumerate([(16, 32, 8, 2048, 2048, 8), (2, 6, 3, 1000, 1024, 5)]):
        print(f"case noalloc call {case}: B={B} H={H} Hkv={Hkv} S={S} splits={splits}", flush=True)
        assert B * H * splits * 130 * 4 <= SCRATCH_BYTES
        host, dev = operands(50 + case, B, H, Hkv, S, cap)
        out = torch.empty_like(dev[0])
        assert noalloc(rbq, dev, S, splits, out) == rbq.RBQ_OK
        want = rbq.attention_decode_int4kv_split(*dev, scale, splits, seq=S)
        torch.cuda.synchronize()
        assert torch.equal(out, want)
        q, kc, ks, vc, vs = host
        rng = np.random.default_rng(case)
        pairs = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(6)]
        check(out, q, kc[:, :, :S], ks[:, :, :S], vc[:, :, :S], vs[:, :, :S], scale, heads=pairs)


def test_noalloc_refuses_partials_beyond_its_array(rbq):
    # 64 x 64 pairs x 4 ranges need 64 * 64 * 4 * 520 bytes > 8 MiB: refused on the host
    # (the buffers do hold that problem, so nothing would be out of bounds even if it ran)
    _, dev = operands(3, 64, 64, 64, 4, 4)
    out = torch.empty_like(dev[0])
    assert noalloc(rbq, dev, 4, 4, out) == rbq.RBQ_ENOTSUP
    assert noalloc(rbq, dev, 4, 3, out) == rbq.RBQ_OK  # 64 * 64 * 3 * 520 bytes fit
    want = rbq.attention_decode_int4kv_split(*dev, 1.0 / math.sqrt(128), 3, seq=4)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
