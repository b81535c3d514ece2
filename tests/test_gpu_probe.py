"""The HBM streaming probe (rbq_hbm_probe, measurement only): it reads and writes exactly
the bytes it is asked to, checked through the value it stores (the xor fold of each lane's
loaded words)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rbq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotation_bit_quantization_fwht_amd as m

    m.lib()
    return m


@pytest.mark.parametrize("rd,wr,blocks", [(32768, 8192, 37), (4096, 4096, 5), (65536, 0, 9)])
def test_probe_moves_the_bytes_it_is_asked_to(rbq, rd, wr, blocks):
    print(f"case hbm_probe read={rd} write={wr} blocks={blocks}", flush=True)
    rng = np.random.default_rng([rd, wr, blocks])
    src_h = rng.integers(0, 2 ** 32, size=blocks * rd // 4, dtype=np.uint32)
    src = torch.from_numpy(src_h.view(np.int32)).cuda()
    nd = blocks * (wr if wr else 16) // 4
    dst = torch.full((nd + 64,), -1, dtype=torch.int32, device="cuda")
    rbq.hbm_probe(src, rd, dst, wr, blocks)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32)
    assert np.all(got[nd:] == 0xFFFFFFFF)  # nothing past the requested bytes
    fold = np.bitwise_xor.reduce(src_h.reshape(blocks, rd // 4096, 256, 4), axis=(1, 3))  # [blocks, 256]
    if wr:
        want = np.broadcast_to(fold[:, None, :, None], (blocks, wr // 4096, 256, 4)).reshape(-1)
        assert np.array_equal(got[:nd], want)
    else:
        assert not np.any(fold == 0x9E3779B9)
        assert np.all(got[:nd] == 0xFFFFFFFF)  # written only when the fold hits the marker
