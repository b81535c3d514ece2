"""CPU tests of the C ABI: the library loads, exports every function include/rbq.h
declares, and rejects invalid arguments on the host (before any HIP call, so these run
without a GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

import oracle
import rotation_bit_quantization_fwht_amd as rbq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rbq.h")


@pytest.fixture(scope="session")
def L():
    if not os.path.exists(rbq.library_path()):
        from rotation_bit_quantization_fwht_amd.build import build

        build()
    return rbq.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(rbq.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", rbq.library_path()], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_status_strings_and_version(L):
    assert L.rbq_status_string(rbq.RBQ_OK) == b"RBQ_OK"
    for s in (rbq.RBQ_EINVAL, rbq.RBQ_ENOTSUP, rbq.RBQ_EHIP):
        assert L.rbq_status_string(s).startswith(b"RBQ_E")
    assert L.rbq_status_string(99) == b"RBQ_UNKNOWN"
    assert b"gfx950" in L.rbq_version()


A16 = ctypes.c_void_p(0x10000)  # a 16-byte aligned fake device address (never dereferenced)
A16b = ctypes.c_void_p(0x20000)
A16c = ctypes.c_void_p(0x30000)
NULL = None


def hq(L, x=A16, dt=rbq.RBQ_BF16, n=4096, tokens=8, stride=4096, codes=A16b, scales=A16c,
       sdt=rbq.RBQ_F16, rot=NULL, flags=rbq.RBQ_PACKED):
    return L.hadamard_quant_int4(x, dt, n, tokens, stride, codes, scales, sdt, rot, flags, NULL)


def test_hadamard_quant_validation(L):
    E = rbq.RBQ_EINVAL
    assert hq(L, tokens=0) == rbq.RBQ_OK
    assert hq(L, x=NULL, codes=NULL, scales=NULL, tokens=0) == rbq.RBQ_OK
    for n in (0, 1, 3, 6, 4095, 65536, -4):
        assert hq(L, n=n, stride=max(n, 1)) == E, n
    assert hq(L, tokens=-1) == E
    assert hq(L, x=NULL) == E
    assert hq(L, codes=NULL) == E
    assert hq(L, scales=NULL) == E
    assert hq(L, stride=4095) == E
    assert hq(L, stride=4100) == E  # 8200-byte rows are not 16-byte aligned
    assert hq(L, x=ctypes.c_void_p(0x10008)) == E
    assert hq(L, codes=ctypes.c_void_p(0x20004)) == E
    assert hq(L, rot=ctypes.c_void_p(0x40004)) == E
    assert hq(L, dt=7) == E
    assert hq(L, sdt=rbq.RBQ_BF16) == E
    assert hq(L, flags=0x80) == E
    assert hq(L, flags=rbq.RBQ_Q_ROTATE_ONLY) == E
    # tiny rows only need element alignment of the row size
    assert hq(L, n=2, stride=2, x=ctypes.c_void_p(0x10004), tokens=0) == rbq.RBQ_OK


def test_signed_validation(L):
    E = rbq.RBQ_EINVAL

    def hs(signs=A16c, flags=rbq.RBQ_PACKED, tokens=8, n=4096, dt=rbq.RBQ_BF16):
        return L.hadamard_quant_int4_signed(A16, dt, n, tokens, n, signs, A16b, A16c, rbq.RBQ_F16, NULL, flags, NULL)

    assert hs(tokens=0) == rbq.RBQ_OK
    assert hs(signs=NULL) == E
    assert hs(signs=ctypes.c_void_p(0x30008)) == E     # not aligned like a row
    assert hs(flags=rbq.RBQ_PACKED | rbq.RBQ_NO_ROTATE) == E
    assert hs(n=4095) == E
    assert hs(dt=9) == E


def kv(L, q=A16, k=A16b, dt=rbq.RBQ_BF16, B=2, H=4, S=16, D=128, qs=None, ks=None, qc=A16c, qsc=A16c,
       kc=A16c, ksc=A16c, sdt=rbq.RBQ_F16, qrot=NULL, flags=0):
    def st(v):
        return (ctypes.c_int64 * 4)(*v) if v is not None else (ctypes.c_int64 * 4)(H * S * D, S * D, D, 1)
    return L.kv_rotate_quant(q, k, dt, B, H, S, D, st(qs), st(ks), qc, qsc, kc, ksc, sdt, qrot, flags, NULL)


def test_kv_validation(L):
    E = rbq.RBQ_EINVAL
    assert kv(L, S=0) == rbq.RBQ_OK
    assert kv(L, D=96) == E
    assert kv(L, D=4) == E
    assert kv(L, dt=rbq.RBQ_F32) == E
    assert kv(L, B=-1) == E
    assert kv(L, q=NULL) == E
    assert kv(L, kc=NULL) == E
    assert kv(L, qc=NULL) == E
    assert kv(L, qc=NULL, qsc=NULL, flags=rbq.RBQ_Q_ROTATE_ONLY) == E  # needs q_rotated
    assert kv(L, qs=(4 * 16 * 128, 16 * 128, 128, 2)) == E  # d stride must be 1
    assert kv(L, qs=(4 * 16 * 128, 16 * 128, 132, 1)) == E  # vector starts not 16-byte aligned
    assert kv(L, flags=rbq.RBQ_PACKED) == E
    # a non-flattenable layout needs head_dim 64/128/256
    assert kv(L, D=512, qs=(16 * 4 * 512, 512, 4 * 512, 1), ks=(16 * 4 * 512, 512, 4 * 512, 1)) == rbq.RBQ_ENOTSUP


def test_gemm_validation(L):
    E, NS = rbq.RBQ_EINVAL, rbq.RBQ_ENOTSUP

    def g(qa=A16, sa=A16b, qw=A16c, sw=A16b, sdt=rbq.RBQ_F16, M=64, N=64, K=4096, out=A16, acc=NULL):
        return L.w4a4_gemm(qa, sa, qw, sw, sdt, M, N, K, out, acc, NULL)

    assert g(M=0) == rbq.RBQ_OK
    assert g(N=0, out=NULL) == rbq.RBQ_OK
    assert g(K=0) == E
    assert g(K=4097) == E
    assert g(M=-1) == E
    assert g(qa=NULL) == E
    assert g(out=NULL) == E
    assert g(sdt=rbq.RBQ_BF16) == E
    assert g(qa=ctypes.c_void_p(0x10001)) == E
    assert g(K=4000) == NS
    assert g(N=60) == NS
    assert g(K=131072) == NS


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("RBQ_LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(rbq, "_lib", None)
    with pytest.raises(rbq.LibraryMissing):
        rbq.lib()


def test_int8_entry_points_validation(L):
    E, NS = rbq.RBQ_EINVAL, rbq.RBQ_ENOTSUP
    hq8 = lambda flags=0, tokens=8: L.hadamard_quant_int8(A16, rbq.RBQ_BF16, 4096, tokens, 4096, A16b, A16c,
                                                          rbq.RBQ_F16, NULL, flags, NULL)
    assert hq8(tokens=0) == rbq.RBQ_OK
    assert hq8(flags=rbq.RBQ_PACKED) == E          # INT8 codes are never packed
    assert hq8(flags=0x80) == E

    def g8(K=4096, N=64, qa=A16):
        return L.w4a8_gemm(qa, A16b, A16c, A16b, rbq.RBQ_F16, 64, N, K, A16, NULL, NULL)

    assert g8(K=4000) == NS
    assert g8(N=60) == NS
    assert g8(K=131072) == NS
    assert g8(qa=NULL) == E
    assert L.w4a8_gemm(A16, A16b, A16c, A16b, rbq.RBQ_F16, 0, 64, 4096, A16, NULL, NULL) == rbq.RBQ_OK



def test_rope_validation(L):
    E, NS = rbq.RBQ_EINVAL, rbq.RBQ_ENOTSUP

    def kr(D=128, cos=A16c, sin=A16c, P=64, pos0=0, S=16, dt=rbq.RBQ_BF16):
        st = (ctypes.c_int64 * 4)(4 * S * D, S * D, D, 1)
        return L.kv_rope_rotate_quant(A16, A16b, dt, 2, 4, S, D, st, st, cos, sin, P, pos0,
                                      A16c, A16c, A16c, A16c, rbq.RBQ_F16, NULL, 0, NULL)

    assert kr(S=0) == rbq.RBQ_OK
    assert kr(cos=NULL) == E
    assert kr(sin=ctypes.c_void_p(0x30004)) == E   # tables must be 16-byte aligned
    assert kr(P=16, pos0=1) == E                     # positions 1..16 exceed 16 table rows
    assert kr(pos0=-1) == E
    assert kr(dt=rbq.RBQ_F32) == E
    assert kr(D=32) == NS                            # RoPE is fused for head_dim 64, 128 and 256


@pytest.fixture(scope="session")
def abi_client(L, tmp_path_factory):
    """tests/host/abi_client.c built with gcc against include/rbq.h and librbq.so."""
    exe = str(tmp_path_factory.mktemp("abi") / "abi_client")
    libdir = os.path.dirname(rbq.library_path())
    libname = os.path.basename(rbq.library_path())
    assert libname.startswith("lib") and libname.endswith(".so")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "host", "abi_client.c"), "-o", exe,
           "-L", libdir, "-l" + libname[3:-3], "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True)
    return exe


def _run_client(exe, mode, **env):
    e = {k: v for k, v in os.environ.items() if not k.startswith("RBQ_")}
    e.update(env)
    return subprocess.run([exe, mode], capture_output=True, text=True, env=e, timeout=120)


def test_plain_c_client_validation(abi_client):
    p = _run_client(abi_client, "validate")
    assert p.returncode == 0, p.stdout + p.stderr
    assert "validate: 0 failure(s)" in p.stdout
    assert "rbq:" not in p.stderr  # no diagnostics unless asked for


def test_fault_injection_reports_launch_failure(abi_client):
    p = _run_client(abi_client, "inject", RBQ_FAULT_INJECT="launch")
    assert p.returncode == 0, p.stdout + p.stderr
    assert "inject: 0 failure(s)" in p.stdout
    # invalid arguments still fail validation first, under injection too
    p = _run_client(abi_client, "validate", RBQ_FAULT_INJECT="launch")
    assert p.returncode == 0, p.stdout + p.stderr


def test_inject_mode_refuses_without_the_switch(abi_client):
    """inject mode passes fake addresses to valid calls: without RBQ_FAULT_INJECT=launch it
    must stop before any call instead of letting them launch."""
    p = _run_client(abi_client, "inject")
    assert p.returncode == 2, p.stdout + p.stderr
    assert "RBQ_FAULT_INJECT=launch is required" in p.stdout
    p = _run_client(abi_client, "inject", RBQ_FAULT_INJECT="other")
    assert p.returncode == 2, p.stdout + p.stderr


def test_dispatch_log(abi_client):
    p = _run_client(abi_client, "inject", RBQ_FAULT_INJECT="launch", RBQ_LOG="1")
    assert p.returncode == 0, p.stdout + p.stderr
    lines = [l for l in p.stderr.splitlines() if l.startswith("rbq: ")]
    assert len(lines) == 17, p.stderr  # one line per valid call, none for rejected ones
    assert lines[0].startswith("rbq: hadamard_quant n=4096 tokens=8 dtype=1 rotate=1 signs=0 int8=0 packed=1")
    assert "signs=1" in lines[1] and "int8=1 packed=0" in lines[2]
    assert "rope=0" in lines[3] and "rope=1" in lines[4]
    assert lines[5].startswith("rbq: hadamard_kron_quant n=5120 m=20 p=256 paley=1 q=19 tokens=8")
    assert lines[6].startswith("rbq: quantize_groups_int4 K=4096 rows=8 group=256")
    assert lines[7].startswith("rbq: w4a8_gemm_grouped M=64 N=64 K=4096 group=256")
    assert lines[8].startswith("rbq: w4a8_gemm_grouped M=64 N=64 K=4096 group=32")
    assert lines[9].startswith("rbq: attention_decode_int4kv B=2 H=8 Hkv=2 S=16")
    assert lines[10].startswith("rbq: w4a4_gemm M=64 N=64 K=4096 tiles=1")
    assert lines[11].startswith("rbq: w4a8_gemm M=64")
    assert lines[12].startswith("rbq: hbm_probe read=65536 write=16384 blocks=8")
    assert lines[13].startswith("rbq: kv_cache_append B=2 H=4 Hkv=2 S=16 D=128 pos0=3 cap=19 rope=1 q=1")
    assert lines[14].startswith("rbq: attention_decode_int4kv_split B=2 H=8 Hkv=2 S=16 cap=16 splits=4")
    assert lines[15].startswith("rbq: kv_cache_append B=2 H=4 Hkv=2 S=16 D=128 pos0=3 cap=19 rope=1 q=0")
    assert lines[16].startswith("rbq: attention_decode_int4kv_split_noalloc B=64 H=64 Hkv=64 S=16 cap=16 splits=3")


def test_kron_validation_and_factor(L):
    E, NS = rbq.RBQ_EINVAL, rbq.RBQ_ENOTSUP

    def hk(n=5120, tokens=8, stride=None, x=A16, flags=rbq.RBQ_PACKED, dt=rbq.RBQ_BF16, sdt=rbq.RBQ_F16):
        return L.hadamard_kron_quant_int4(x, dt, n, tokens, stride or n, A16b, A16c, sdt, NULL, flags, NULL)

    assert hk(tokens=0) == rbq.RBQ_OK
    assert hk(n=16640) == NS          # 65 * 256: no construction of order 260 or below
    assert hk(n=172 * 128) == NS      # the row buffer and the table exceed a workgroup's LDS
    assert hk(n=252 * 32) == NS       # likewise for Paley order 252 with p = 32
    assert hk(n=12 * 8) == NS         # p = 8 < 16
    assert hk(n=6) == NS              # no factor
    assert hk(n=40000) == E
    assert hk(tokens=-1) == E
    assert hk(x=NULL) == E
    assert hk(stride=5119) == E
    assert hk(stride=5124) == E       # 10248-byte rows are not 16-byte aligned
    assert hk(x=ctypes.c_void_p(0x10008)) == E
    assert hk(flags=rbq.RBQ_NO_ROTATE) == E
    assert hk(dt=9) == E
    assert hk(sdt=rbq.RBQ_BF16) == E
    # the library's factor rule agrees with the oracle's on every length up to 40000
    for n in range(1, 40001):
        want = oracle.kron_factor(n)
        got = rbq.kron_factor(n)
        assert got == want, n


def test_group_entry_points_validation(L):
    E, NS = rbq.RBQ_EINVAL, rbq.RBQ_ENOTSUP

    def qg(K=4096, rows=8, stride=None, group=256, y=A16, dt=rbq.RBQ_F32, flags=rbq.RBQ_PACKED, sdt=rbq.RBQ_F16):
        return L.quantize_groups_int4(y, dt, K, rows, stride or K, group, A16b, A16c, sdt, flags, NULL)

    assert qg(rows=0) == rbq.RBQ_OK
    for g in (16, 48, 8192, 4096 * 2):
        assert qg(group=g, K=8192) == E, g
    assert qg(group=512, K=768) == E        # must divide K
    assert qg(y=NULL) == E
    assert qg(stride=4095) == E
    assert qg(y=ctypes.c_void_p(0x10004)) == E
    assert qg(flags=rbq.RBQ_NO_ROTATE) == E
    assert qg(sdt=rbq.RBQ_BF16) == E

    def gg(group=256, K=4096, N=64, qa=A16):
        return L.w4a8_gemm_grouped(qa, A16b, A16c, A16b, rbq.RBQ_F16, group, 64, N, K, A16, NULL)

    assert L.w4a8_gemm_grouped(A16, A16b, A16c, A16b, rbq.RBQ_F16, 256, 0, 64, 4096, A16, NULL) == rbq.RBQ_OK
    assert gg(group=48) == E
    assert gg(group=8192) == E
    assert gg(group=16) == E                # below the smallest group of 32 codes
    assert gg(group=32, K=4000) == NS       # (valid groups are launched, so only failing shapes here)
    assert gg(group=64, N=60) == NS
    assert gg(K=4000) == NS
    assert gg(N=60) == NS
    assert gg(qa=NULL) == E


def test_attention_validation(L):
    E, NS = rbq.RBQ_EINVAL, rbq.RBQ_ENOTSUP

    def at(q=A16, qdt=rbq.RBQ_BF16, sdt=rbq.RBQ_F16, B=2, H=8, Hkv=2, S=16, cap=16, D=128, scale=0.1):
        return L.attention_decode_int4kv(q, qdt, A16b, A16c, A16b, A16c, sdt, B, H, Hkv, S, cap, D, scale, A16, NULL)

    assert at(B=0) == rbq.RBQ_OK
    assert at(S=0) == E
    assert at(cap=8) == E                    # capacity below the sequence
    assert at(H=6, Hkv=4) == E               # heads not a multiple of kv heads
    assert at(qdt=rbq.RBQ_F32) == E
    assert at(sdt=rbq.RBQ_BF16) == E
    assert at(q=NULL) == E
    assert at(q=ctypes.c_void_p(0x10008)) == E
    assert at(scale=float("nan")) == E
    assert at(D=64) == NS
    assert at(S=1 << 26, cap=1 << 26) == NS  # one head's codes past 32-bit byte offsets
    assert at(S=16, cap=(1 << 30) + 1) == NS


def test_attention_split_validation(L):
    E, NS = rbq.RBQ_EINVAL, rbq.RBQ_ENOTSUP
    need = 2 * 8 * 4 * 130 * 4

    def sp(splits=4, ws=A16b, ws_bytes=need, B=2, H=8, Hkv=2, S=16, D=128):
        return L.attention_decode_int4kv_split(A16, rbq.RBQ_BF16, A16b, A16c, A16b, A16c, rbq.RBQ_F16, B, H, Hkv, S,
                                               S, D, 0.1, splits, ws, ws_bytes, A16, NULL)

    assert sp(B=0, ws=NULL, ws_bytes=0) == rbq.RBQ_OK
    assert sp(splits=0) == E
    assert sp(splits=4097) == E
    assert sp(ws=NULL) == E
    assert sp(ws=ctypes.c_void_p(0x20008)) == E
    assert sp(ws_bytes=need - 1) == E
    assert sp(D=256) == NS
    assert sp(H=6, Hkv=4) == E
    n = ctypes.c_int64(0)
    assert L.rbq_attention_split_workspace_bytes(2, 8, 4, ctypes.byref(n)) == rbq.RBQ_OK and n.value == need
    assert L.rbq_attention_split_workspace_bytes(-1, 8, 4, ctypes.byref(n)) == E
    assert rbq.attention_split_workspace_bytes(16, 32, 8) == 16 * 32 * 8 * 130 * 4
