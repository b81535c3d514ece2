"""Thin Python binding of librbq.so, the C-ABI HIP library for MI355X (gfx950).

The calls have the same names and meaning as the C functions declared in
``include/rbq.h``:

* ``hadamard_quant_int4`` -- Sylvester-Hadamard rotation per row fused with per-row
  symmetric INT4 absmax quantization (round half to even), codes packed two per byte
  (optionally the randomized transform with a +-1 diagonal);
* ``hadamard_kron_quant_int4`` -- the same for row lengths that are not powers of two,
  rotated by the Kronecker product of a Paley or Goethals-Seidel matrix with a Sylvester matrix
  (``kron_factor`` reports the order of the small factor);
* ``hadamard_quant_int8`` -- the same with INT8 codes;
* ``kv_rotate_quant`` -- the same per (batch, head, token) vector of post-RoPE Q and K
  (optionally with RoPE applied first);
* ``w4a4_gemm`` / ``w4a8_gemm`` -- the GEMMs on packed INT4 weight codes with int32
  accumulation and a bf16 dequantization epilogue;
* ``quantize_groups_int4`` / ``w4a8_gemm_grouped`` -- group-wise weight scales: the
  quantizer (one scale per run of ``group`` elements) and the W4A8 GEMM that consumes it;
* ``attention_decode_int4kv`` -- decode attention over the INT4 key/value cache;
  ``attention_decode_int4kv_split`` the same with each sequence cut into ranges taken by
  separate workgroups, their partials combined through a caller's workspace
  (``attention_decode_int4kv_split_noalloc``: through the library's fixed device array,
  for callers that cannot allocate).

This module only marshals arguments: it takes ``torch.Tensor`` objects that live in GPU
memory, allocates outputs with torch when the caller does not pass them, and hands raw
device pointers and the current HIP stream to the library. Every step of the computation
runs in the library's kernels. If the library is missing the calls raise; there is no
fallback.
"""

import ctypes
import os

__all__ = [
    "RBQError",
    "LibraryMissing",
    "lib",
    "library_path",
    "hadamard_quant_int4",
    "hadamard_quant_int8",
    "hadamard_kron_quant_int4",
    "kron_factor",
    "kv_rotate_quant",
    "kv_cache_append_int4",
    "w4a4_gemm",
    "w4a8_gemm",
    "w4a8_gemm_grouped",
    "quantize_groups_int4",
    "attention_decode_int4kv",
    "attention_decode_int4kv_split",
    "attention_decode_int4kv_split_noalloc",
    "attention_split_workspace_bytes",
    "hbm_probe",
    "RBQ_OK",
    "RBQ_EINVAL",
    "RBQ_ENOTSUP",
    "RBQ_EHIP",
    "RBQ_F32",
    "RBQ_BF16",
    "RBQ_F16",
    "RBQ_PACKED",
    "RBQ_NO_ROTATE",
    "RBQ_Q_ROTATE_ONLY",
    "EXPORTED_SYMBOLS",
]

RBQ_OK, RBQ_EINVAL, RBQ_ENOTSUP, RBQ_EHIP = 0, 1, 2, 3
RBQ_F32, RBQ_BF16, RBQ_F16 = 0, 1, 2
RBQ_PACKED, RBQ_NO_ROTATE, RBQ_Q_ROTATE_ONLY = 1, 2, 4

EXPORTED_SYMBOLS = (
    "hadamard_quant_int4",
    "hadamard_quant_int4_signed",
    "hadamard_quant_int8",
    "hadamard_kron_quant_int4",
    "rbq_kron_factor",
    "kv_rotate_quant",
    "kv_rope_rotate_quant",
    "kv_cache_append_int4",
    "w4a4_gemm",
    "w4a8_gemm",
    "w4a8_gemm_grouped",
    "quantize_groups_int4",
    "attention_decode_int4kv",
    "attention_decode_int4kv_split",
    "attention_decode_int4kv_split_noalloc",
    "rbq_attention_split_workspace_bytes",
    "rbq_hbm_probe",
    "rbq_status_string",
    "rbq_version",
)

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.environ.get("RBQ_LIBRARY", os.path.join(_HERE, "librbq.so"))


class LibraryMissing(RuntimeError):
    pass


class RBQError(RuntimeError):
    def __init__(self, func, status, message):
        super().__init__(f"{func}: {message} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load librbq.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise LibraryMissing(
            f"{path} is not built; run rotation_bit_quantization_fwht_amd.build.build() "
            "(hipcc --offload-arch=gfx950). There is no CPU fallback."
        )
    L = ctypes.CDLL(path)
    vp, i64, ci, cu = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    p64 = ctypes.POINTER(ctypes.c_int64)
    L.hadamard_quant_int4.argtypes = [vp, ci, i64, i64, i64, vp, vp, ci, vp, cu, vp]
    L.hadamard_quant_int4.restype = ci
    L.hadamard_quant_int4_signed.argtypes = [vp, ci, i64, i64, i64, vp, vp, vp, ci, vp, cu, vp]
    L.hadamard_quant_int4_signed.restype = ci
    L.hadamard_quant_int8.argtypes = [vp, ci, i64, i64, i64, vp, vp, ci, vp, cu, vp]
    L.hadamard_quant_int8.restype = ci
    L.hadamard_kron_quant_int4.argtypes = [vp, ci, i64, i64, i64, vp, vp, ci, vp, cu, vp]
    L.hadamard_kron_quant_int4.restype = ci
    L.rbq_kron_factor.argtypes = [i64, p64]
    L.rbq_kron_factor.restype = ci
    L.kv_rotate_quant.argtypes = [vp, vp, ci, i64, i64, i64, i64, p64, p64, vp, vp, vp, vp, ci, vp, cu, vp]
    L.kv_rotate_quant.restype = ci
    L.kv_rope_rotate_quant.argtypes = [vp, vp, ci, i64, i64, i64, i64, p64, p64, vp, vp, i64, i64,
                                       vp, vp, vp, vp, ci, vp, cu, vp]
    L.kv_rope_rotate_quant.restype = ci
    L.kv_cache_append_int4.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, p64, p64, p64, vp, vp, i64, i64,
                                       i64, vp, vp, vp, vp, vp, ci, vp]
    L.kv_cache_append_int4.restype = ci
    L.w4a4_gemm.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, vp, vp, vp]
    L.w4a4_gemm.restype = ci
    L.w4a8_gemm.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, vp, vp, vp]
    L.w4a8_gemm.restype = ci
    L.w4a8_gemm_grouped.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, vp, vp]
    L.w4a8_gemm_grouped.restype = ci
    L.quantize_groups_int4.argtypes = [vp, ci, i64, i64, i64, i64, vp, vp, ci, cu, vp]
    L.quantize_groups_int4.restype = ci
    L.attention_decode_int4kv.argtypes = [vp, ci, vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64,
                                          ctypes.c_float, vp, vp]
    L.attention_decode_int4kv.restype = ci
    L.attention_decode_int4kv_split.argtypes = [vp, ci, vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64,
                                                ctypes.c_float, i64, vp, i64, vp, vp]
    L.attention_decode_int4kv_split.restype = ci
    L.attention_decode_int4kv_split_noalloc.argtypes = [vp, ci, vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64,
                                                        ctypes.c_float, i64, vp, vp]
    L.attention_decode_int4kv_split_noalloc.restype = ci
    L.rbq_attention_split_workspace_bytes.argtypes = [i64, i64, i64, p64]
    L.rbq_attention_split_workspace_bytes.restype = ci
    L.rbq_hbm_probe.argtypes = [vp, i64, vp, i64, i64, vp]
    L.rbq_hbm_probe.restype = ci
    L.rbq_status_string.argtypes = [ci]
    L.rbq_status_string.restype = ctypes.c_char_p
    L.rbq_version.argtypes = []
    L.rbq_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(func, status):
    if status != RBQ_OK:
        msg = lib().rbq_status_string(status).decode()
        raise RBQError(func, status, msg)


def _torch():
    import torch

    return torch


_DTYPE_CODES = None


def _dtype_code(t):
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        torch = _torch()
        _DTYPE_CODES = {torch.float32: RBQ_F32, torch.bfloat16: RBQ_BF16, torch.float16: RBQ_F16}
    code = _DTYPE_CODES.get(t)
    if code is None:
        raise TypeError(f"unsupported dtype {t}")
    return code


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    """The HIP stream to launch on: ``stream`` if given, else torch's current stream on
    ``device``. The current stream's handle is read with torch's raw query where it has one
    (a few hundredths of a microsecond, against about 2 us for building a Stream object)."""
    torch = _torch()
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return ctypes.c_void_p(raw(device.index if device.index is not None else torch.cuda.current_device()))
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("rbq kernels take GPU tensors only")


def _require_buffer(name, t, shape, dtypes, device):
    """A caller-provided output must be a contiguous tensor of exactly this shape and one
    of these dtypes on the input's device: the kernels write it without bounds checks."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous {'/'.join(str(d) for d in dtypes)} tensor of shape "
                         f"{tuple(shape)} on {device}; got {t.dtype} {tuple(t.shape)} on {t.device}")


def hadamard_quant_int4(x, *, scale_dtype=None, packed=True, rotate=True, codes=None, scales=None,
                        rotated=None, return_rotated=False, signs=None, stream=None):
    """Rotate every row of ``x`` [tokens, n] (last dim contiguous) by H_n / sqrt(n) and
    quantize it to INT4 with one absmax scale per row.

    Returns ``(codes, scales)`` -- codes uint8 [tokens, n/2] (packed) or int8
    [tokens, n]; scales [tokens] in ``scale_dtype`` (default float16) -- plus the float
    rotated rows when ``return_rotated`` (or a ``rotated`` buffer) is given.
    ``signs`` ([n] of +-1 in x's dtype) selects the randomized transform
    H_n diag(signs) / sqrt(n) (entry point hadamard_quant_int4_signed).
    """
    torch = _torch()
    _require_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with a contiguous last dimension")
    tokens, n = x.shape
    scale_dtype = torch.float16 if scale_dtype is None else scale_dtype
    dev = x.device
    if codes is None:
        codes = torch.empty((tokens, n // 2 if packed else n), dtype=torch.uint8 if packed else torch.int8, device=dev)
    if scales is None:
        scales = torch.empty((tokens,), dtype=scale_dtype, device=dev)
    if rotated is None and return_rotated:
        rotated = torch.empty((tokens, n), dtype=torch.float32, device=dev)
    _require_cuda(codes, scales, rotated)
    _require_buffer("codes", codes, (tokens, n // 2) if packed else (tokens, n),
                    (torch.uint8,) if packed else (torch.int8, torch.uint8), dev)
    _require_buffer("scales", scales, (tokens,), (torch.float16, torch.float32), dev)
    _require_buffer("rotated", rotated, (tokens, n), (torch.float32,), dev)
    flags = (RBQ_PACKED if packed else 0) | (0 if rotate else RBQ_NO_ROTATE)
    if signs is not None:
        _require_cuda(signs)
        _require_buffer("signs", signs, (n,), (x.dtype,), dev)
        st = lib().hadamard_quant_int4_signed(
            _ptr(x), _dtype_code(x.dtype), n, tokens, x.stride(0) if tokens > 0 else n, _ptr(signs),
            _ptr(codes), _ptr(scales), _dtype_code(scales.dtype), _ptr(rotated), flags, _stream(stream, dev),
        )
        _check("hadamard_quant_int4_signed", st)
    else:
        st = lib().hadamard_quant_int4(
            _ptr(x), _dtype_code(x.dtype), n, tokens, x.stride(0) if tokens > 0 else n,
            _ptr(codes), _ptr(scales), _dtype_code(scales.dtype), _ptr(rotated), flags, _stream(stream, dev),
        )
        _check("hadamard_quant_int4", st)
    if rotated is not None:
        return codes, scales, rotated
    return codes, scales


def kron_factor(n):
    """Order m of the small factor used for row length n (1 for a power of two), or None
    when the library has no factorization for n."""
    m = ctypes.c_int64(0)
    st = lib().rbq_kron_factor(int(n), ctypes.byref(m))
    if st == RBQ_ENOTSUP:
        return None
    _check("rbq_kron_factor", st)
    return m.value


def hadamard_kron_quant_int4(x, *, scale_dtype=None, packed=True, codes=None, scales=None, rotated=None,
                             return_rotated=False, stream=None):
    """As ``hadamard_quant_int4`` for any supported row length n = m * p: every row of
    ``x`` [tokens, n] is rotated by (H_m (x) H_p) / sqrt(n) and quantized to INT4 with
    one absmax scale per row. Returns ``(codes, scales)`` (+ the rotated rows when
    requested)."""
    torch = _torch()
    _require_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with a contiguous last dimension")
    tokens, n = x.shape
    scale_dtype = torch.float16 if scale_dtype is None else scale_dtype
    dev = x.device
    if codes is None:
        codes = torch.empty((tokens, n // 2 if packed else n), dtype=torch.uint8 if packed else torch.int8, device=dev)
    if scales is None:
        scales = torch.empty((tokens,), dtype=scale_dtype, device=dev)
    if rotated is None and return_rotated:
        rotated = torch.empty((tokens, n), dtype=torch.float32, device=dev)
    _require_cuda(codes, scales, rotated)
    _require_buffer("codes", codes, (tokens, n // 2) if packed else (tokens, n),
                    (torch.uint8,) if packed else (torch.int8, torch.uint8), dev)
    _require_buffer("scales", scales, (tokens,), (torch.float16, torch.float32), dev)
    _require_buffer("rotated", rotated, (tokens, n), (torch.float32,), dev)
    st = lib().hadamard_kron_quant_int4(
        _ptr(x), _dtype_code(x.dtype), n, tokens, x.stride(0) if tokens > 0 else n,
        _ptr(codes), _ptr(scales), _dtype_code(scales.dtype), _ptr(rotated), RBQ_PACKED if packed else 0,
        _stream(stream, dev),
    )
    _check("hadamard_kron_quant_int4", st)
    if rotated is not None:
        return codes, scales, rotated
    return codes, scales


def hadamard_quant_int8(x, *, scale_dtype=None, rotate=True, codes=None, scales=None, rotated=None,
                        return_rotated=False, stream=None):
    """As ``hadamard_quant_int4`` with INT8 codes (scale max/127, int8 [tokens, n]) for
    W4A8 layers. Returns ``(codes, scales)`` (+ the rotated rows when requested)."""
    torch = _torch()
    _require_cuda(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with a contiguous last dimension")
    tokens, n = x.shape
    scale_dtype = torch.float16 if scale_dtype is None else scale_dtype
    dev = x.device
    if codes is None:
        codes = torch.empty((tokens, n), dtype=torch.int8, device=dev)
    if scales is None:
        scales = torch.empty((tokens,), dtype=scale_dtype, device=dev)
    if rotated is None and return_rotated:
        rotated = torch.empty((tokens, n), dtype=torch.float32, device=dev)
    _require_cuda(codes, scales, rotated)
    _require_buffer("codes", codes, (tokens, n), (torch.int8,), dev)
    _require_buffer("scales", scales, (tokens,), (torch.float16, torch.float32), dev)
    _require_buffer("rotated", rotated, (tokens, n), (torch.float32,), dev)
    st = lib().hadamard_quant_int8(
        _ptr(x), _dtype_code(x.dtype), n, tokens, x.stride(0) if tokens > 0 else n,
        _ptr(codes), _ptr(scales), _dtype_code(scales.dtype), _ptr(rotated),
        0 if rotate else RBQ_NO_ROTATE, _stream(stream, dev),
    )
    _check("hadamard_quant_int8", st)
    if rotated is not None:
        return codes, scales, rotated
    return codes, scales


def kv_rotate_quant(q, k, *, scale_dtype=None, q_rotate_only=False, q_codes=None, q_scales=None,
                    k_codes=None, k_scales=None, q_rotated=None, rope_cos=None, rope_sin=None,
                    rope_pos0=0, stream=None):
    """R3 on post-RoPE ``q`` and ``k`` [B, H, S, D] (bf16/fp16, D contiguous): rotate every
    head vector by H_D / sqrt(D) and quantize it to packed INT4 with one scale per vector.

    Returns a dict with ``k_codes`` [B,H,S,D/2], ``k_scales`` [B,H,S] and either
    ``q_codes``/``q_scales`` or, with ``q_rotate_only``, ``q_rotated`` [B,H,S,D].
    With ``rope_cos``/``rope_sin`` (float32 [positions, D/2]) q and k are pre-RoPE and the
    half-split rotary embedding at positions rope_pos0 + s is applied first
    (entry point kv_rope_rotate_quant).
    """
    torch = _torch()
    _require_cuda(q, k)
    if q.dim() != 4 or k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must be [B, H, S, D] tensors of one shape and dtype")
    B, H, S, D = q.shape
    scale_dtype = torch.float16 if scale_dtype is None else scale_dtype
    dev = q.device
    out = {}
    if q_rotate_only:
        if q_rotated is None:
            q_rotated = torch.empty((B, H, S, D), dtype=q.dtype, device=dev)
        out["q_rotated"] = q_rotated
    else:
        if q_codes is None:
            q_codes = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=dev)
        if q_scales is None:
            q_scales = torch.empty((B, H, S), dtype=scale_dtype, device=dev)
        out["q_codes"], out["q_scales"] = q_codes, q_scales
    if k_codes is None:
        k_codes = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=dev)
    if k_scales is None:
        k_scales = torch.empty((B, H, S), dtype=scale_dtype, device=dev)
    out["k_codes"], out["k_scales"] = k_codes, k_scales
    _require_cuda(q_codes, q_scales, k_codes, k_scales, q_rotated)
    _require_buffer("q_codes", q_codes, (B, H, S, D // 2), (torch.uint8,), dev)
    _require_buffer("k_codes", k_codes, (B, H, S, D // 2), (torch.uint8,), dev)
    _require_buffer("q_scales", q_scales, (B, H, S), (k_scales.dtype,), dev)
    _require_buffer("k_scales", k_scales, (B, H, S), (torch.float16, torch.float32), dev)
    _require_buffer("q_rotated", q_rotated, (B, H, S, D), (q.dtype,), dev)
    qs = (ctypes.c_int64 * 4)(*q.stride())
    ks = (ctypes.c_int64 * 4)(*k.stride())
    sdt = _dtype_code(k_scales.dtype)
    flags = RBQ_Q_ROTATE_ONLY if q_rotate_only else 0
    if rope_cos is not None or rope_sin is not None:
        if rope_cos is None or rope_sin is None:
            raise ValueError("rope_cos and rope_sin go together")
        _require_cuda(rope_cos, rope_sin)
        P = rope_cos.shape[0] if rope_cos.dim() == 2 else -1
        _require_buffer("rope_cos", rope_cos, (P, D // 2), (torch.float32,), dev)
        _require_buffer("rope_sin", rope_sin, (P, D // 2), (torch.float32,), dev)
        st = lib().kv_rope_rotate_quant(
            _ptr(q), _ptr(k), _dtype_code(q.dtype), B, H, S, D, qs, ks, _ptr(rope_cos), _ptr(rope_sin),
            P, int(rope_pos0), _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), sdt,
            _ptr(q_rotated), flags, _stream(stream, dev),
        )
        _check("kv_rope_rotate_quant", st)
        return out
    st = lib().kv_rotate_quant(
        _ptr(q), _ptr(k), _dtype_code(q.dtype), B, H, S, D, qs, ks,
        _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), sdt, _ptr(q_rotated),
        flags, _stream(stream, dev),
    )
    _check("kv_rotate_quant", st)
    return out


def kv_cache_append_int4(k, v, k_cache, k_cache_scales, v_cache, v_cache_scales, pos0, *, q=None, q_rotated=None,
                         rope_cos=None, rope_sin=None, stream=None):
    """Append one step's keys and values to the INT4 cache: ``k``, ``v`` [B, Hkv, S, D]
    (bf16/fp16, D contiguous, any other strides) go through RoPE at positions pos0 + s
    (when the float32 tables ``rope_cos``/``rope_sin`` [positions, D/2] are given) and, for
    the keys, the rotation H_D / sqrt(D), are quantized to INT4 and written to rows
    pos0 .. pos0 + S - 1 of ``k_cache``/``v_cache`` uint8 [B, Hkv, cap, D/2] and
    ``k_cache_scales``/``v_cache_scales`` [B, Hkv, cap]. With ``q`` [B, H, S, D] the queries
    get RoPE and the rotation and are returned in q's dtype (``q_rotated``, allocated if not
    given); otherwise None is returned."""
    torch = _torch()
    _require_cuda(k, v, k_cache, k_cache_scales, v_cache, v_cache_scales)
    if k.dim() != 4 or v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must be [B, Hkv, S, D] tensors of one shape and dtype")
    B, Hkv, S, D = k.shape
    cap = k_cache.shape[2] if k_cache.dim() == 4 else -1
    dev = k.device
    _require_buffer("k_cache", k_cache, (B, Hkv, cap, D // 2), (torch.uint8,), dev)
    _require_buffer("v_cache", v_cache, (B, Hkv, cap, D // 2), (torch.uint8,), dev)
    _require_buffer("k_cache_scales", k_cache_scales, (B, Hkv, cap), (torch.float16, torch.float32), dev)
    _require_buffer("v_cache_scales", v_cache_scales, (B, Hkv, cap), (k_cache_scales.dtype,), dev)
    H = Hkv
    if q is not None:
        _require_cuda(q)
        if q.dim() != 4 or q.shape[0] != B or q.shape[2] != S or q.shape[3] != D or q.dtype != k.dtype:
            raise ValueError("q must be [B, H, S, D] in k's dtype")
        H = q.shape[1]
        if q_rotated is None:
            q_rotated = torch.empty((B, H, S, D), dtype=q.dtype, device=dev)
        _require_buffer("q_rotated", q_rotated, (B, H, S, D), (q.dtype,), dev)
    elif q_rotated is not None:
        raise ValueError("q_rotated needs q")
    P = 0
    if rope_cos is not None or rope_sin is not None:
        if rope_cos is None or rope_sin is None:
            raise ValueError("rope_cos and rope_sin go together")
        _require_cuda(rope_cos, rope_sin)
        P = rope_cos.shape[0] if rope_cos.dim() == 2 else -1
        _require_buffer("rope_cos", rope_cos, (P, D // 2), (torch.float32,), dev)
        _require_buffer("rope_sin", rope_sin, (P, D // 2), (torch.float32,), dev)
    qs = (ctypes.c_int64 * 4)(*q.stride()) if q is not None else None
    ks = (ctypes.c_int64 * 4)(*k.stride())
    vs = (ctypes.c_int64 * 4)(*v.stride())
    st = lib().kv_cache_append_int4(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(k.dtype), B, H, Hkv, S, D, qs, ks, vs, _ptr(rope_cos),
        _ptr(rope_sin), P, int(pos0), cap, _ptr(q_rotated), _ptr(k_cache), _ptr(k_cache_scales), _ptr(v_cache),
        _ptr(v_cache_scales), _dtype_code(k_cache_scales.dtype), _stream(stream, dev))
    _check("kv_cache_append_int4", st)
    return q_rotated


def w4a4_gemm(qa, sa, qw, sw, *, out=None, acc=None, return_acc=False, stream=None):
    """out[m, n] = bf16(sa[m] * sw[n] * sum_k qa[m, k] qw[n, k]) on packed INT4 codes.

    qa uint8 [M, K/2], qw uint8 [N, K/2] (contiguous), sa [M], sw [N] (fp16 or fp32, same
    dtype). Returns ``out`` (bf16 [M, N]), plus the int32 accumulators when requested.
    """
    torch = _torch()
    _require_cuda(qa, sa, qw, sw)
    if qa.dim() != 2 or qw.dim() != 2 or qa.shape[1] != qw.shape[1]:
        raise ValueError("qa must be [M, K/2] and qw [N, K/2]")
    if not (qa.is_contiguous() and qw.is_contiguous() and sa.is_contiguous() and sw.is_contiguous()):
        raise ValueError("operands must be contiguous")
    if sa.dtype != sw.dtype:
        raise ValueError("sa and sw must share a dtype")
    M, N, K = qa.shape[0], qw.shape[0], 2 * qa.shape[1]
    dev = qa.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if acc is None and return_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    _require_cuda(out, acc)
    if qa.dtype != torch.uint8 or qw.dtype != torch.uint8:
        raise ValueError("qa and qw must be uint8 packed codes")
    if tuple(sa.shape) != (M,) or tuple(sw.shape) != (N,):
        raise ValueError("sa must be [M] and sw [N]")
    _require_buffer("out", out, (M, N), (torch.bfloat16,), dev)
    _require_buffer("acc", acc, (M, N), (torch.int32,), dev)
    st = lib().w4a4_gemm(
        _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _dtype_code(sa.dtype), M, N, K, _ptr(out), _ptr(acc),
        _stream(stream, dev),
    )
    _check("w4a4_gemm", st)
    if acc is not None:
        return out, acc
    return out


def w4a8_gemm(qa, sa, qw, sw, *, out=None, acc=None, return_acc=False, stream=None):
    """out[m, n] = bf16(sa[m] * sw[n] * sum_k qa[m, k] qw[n, k]) with INT8 activation codes
    qa int8 [M, K] and packed INT4 weight codes qw uint8 [N, K/2] (contiguous); sa [M],
    sw [N] share an fp16/fp32 dtype. Returns ``out`` (+ the int32 sums when requested)."""
    torch = _torch()
    _require_cuda(qa, sa, qw, sw)
    if qa.dim() != 2 or qw.dim() != 2 or qa.shape[1] != 2 * qw.shape[1]:
        raise ValueError("qa must be [M, K] and qw [N, K/2]")
    if not (qa.is_contiguous() and qw.is_contiguous() and sa.is_contiguous() and sw.is_contiguous()):
        raise ValueError("operands must be contiguous")
    if qa.dtype != torch.int8 or qw.dtype != torch.uint8:
        raise ValueError("qa must be int8 codes and qw uint8 packed codes")
    if sa.dtype != sw.dtype:
        raise ValueError("sa and sw must share a dtype")
    M, N, K = qa.shape[0], qw.shape[0], qa.shape[1]
    if tuple(sa.shape) != (M,) or tuple(sw.shape) != (N,):
        raise ValueError("sa must be [M] and sw [N]")
    dev = qa.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if acc is None and return_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=dev)
    _require_cuda(out, acc)
    _require_buffer("out", out, (M, N), (torch.bfloat16,), dev)
    _require_buffer("acc", acc, (M, N), (torch.int32,), dev)
    st = lib().w4a8_gemm(
        _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _dtype_code(sa.dtype), M, N, K, _ptr(out), _ptr(acc),
        _stream(stream, dev),
    )
    _check("w4a8_gemm", st)
    if acc is not None:
        return out, acc
    return out



def quantize_groups_int4(y, group, *, scale_dtype=None, packed=True, codes=None, scales=None, stream=None):
    """Group-wise INT4 quantization of rows ``y`` [rows, K] (already in the rotated basis):
    one absmax scale per run of ``group`` consecutive elements. Returns ``(codes, scales)``
    -- codes uint8 [rows, K/2] (packed) or int8 [rows, K], scales [rows, K/group]."""
    torch = _torch()
    _require_cuda(y)
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be a 2-D tensor with a contiguous last dimension")
    rows, K = y.shape
    if group <= 0 or K % group:
        raise ValueError("group must divide the row length")
    scale_dtype = torch.float16 if scale_dtype is None else scale_dtype
    dev = y.device
    if codes is None:
        codes = torch.empty((rows, K // 2 if packed else K), dtype=torch.uint8 if packed else torch.int8, device=dev)
    if scales is None:
        scales = torch.empty((rows, K // group), dtype=scale_dtype, device=dev)
    _require_cuda(codes, scales)
    _require_buffer("codes", codes, (rows, K // 2) if packed else (rows, K),
                    (torch.uint8,) if packed else (torch.int8, torch.uint8), dev)
    _require_buffer("scales", scales, (rows, K // group), (torch.float16, torch.float32), dev)
    st = lib().quantize_groups_int4(
        _ptr(y), _dtype_code(y.dtype), K, rows, y.stride(0) if rows > 0 else K, int(group),
        _ptr(codes), _ptr(scales), _dtype_code(scales.dtype), RBQ_PACKED if packed else 0, _stream(stream, dev))
    _check("quantize_groups_int4", st)
    return codes, scales


def w4a8_gemm_grouped(qa, sa, qw, sw, group, *, out=None, stream=None):
    """out[m, n] = bf16(sa[m] * sum_g sw[n, g] * sum_{k in group g} qa[m, k] qw[n, k]) with
    INT8 activation codes qa int8 [M, K], packed INT4 weight codes qw uint8 [N, K/2] and
    group-wise weight scales sw [N, K/group] (same dtype as sa [M])."""
    torch = _torch()
    _require_cuda(qa, sa, qw, sw)
    M, K = qa.shape
    N = qw.shape[0]
    if qw.shape != (N, K // 2) or group <= 0 or K % group:
        raise ValueError("qa must be [M, K], qw [N, K/2] and group must divide K")
    dev = qa.device
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _require_buffer("qa", qa, (M, K), (torch.int8,), dev)
    _require_buffer("qw", qw, (N, K // 2), (torch.uint8,), dev)
    _require_buffer("sa", sa, (M,), (sw.dtype,), dev)
    _require_buffer("sw", sw, (N, K // group), (torch.float16, torch.float32), dev)
    _require_buffer("out", out, (M, N), (torch.bfloat16,), dev)
    st = lib().w4a8_gemm_grouped(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _dtype_code(sw.dtype), int(group),
                                 M, N, K, _ptr(out), _stream(stream, dev))
    _check("w4a8_gemm_grouped", st)
    return out


def attention_decode_int4kv(q, k_codes, k_scales, v_codes, v_scales, softmax_scale, *, seq=None, out=None,
                            stream=None):
    """Decode attention of q [B, H, 128] (the R3-rotated query) over the INT4 cache:
    k_codes / v_codes uint8 [B, Hkv, S_cap, 64], k_scales / v_scales [B, Hkv, S_cap];
    the first ``seq`` tokens (default S_cap) are attended. Returns out [B, H, 128] in q's
    dtype."""
    (B, H, Hkv, seq, S_cap, D), out = _attention_operands(q, k_codes, k_scales, v_codes, v_scales, seq, out)
    st = lib().attention_decode_int4kv(_ptr(q), _dtype_code(q.dtype), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                       _ptr(v_scales), _dtype_code(k_scales.dtype), B, H, Hkv, seq, S_cap, D,
                                       float(softmax_scale), _ptr(out), _stream(stream, q.device))
    _check("attention_decode_int4kv", st)
    return out


def _attention_operands(q, k_codes, k_scales, v_codes, v_scales, seq, out):
    torch = _torch()
    _require_cuda(q, k_codes, k_scales, v_codes, v_scales)
    B, H, D = q.shape
    _, Hkv, S_cap, half = k_codes.shape
    seq = S_cap if seq is None else int(seq)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    _require_buffer("q", q, (B, H, D), (torch.bfloat16, torch.float16), dev)
    for name, t, shape in (("k_codes", k_codes, (B, Hkv, S_cap, D // 2)), ("v_codes", v_codes, (B, Hkv, S_cap, D // 2))):
        _require_buffer(name, t, shape, (torch.uint8,), dev)
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        _require_buffer(name, t, (B, Hkv, S_cap), (torch.float16, torch.float32), dev)
    if v_scales.dtype != k_scales.dtype:
        raise ValueError("k_scales and v_scales must share a dtype")
    _require_buffer("out", out, (B, H, D), (q.dtype,), dev)
    return (B, H, Hkv, seq, S_cap, D), out


def attention_split_workspace_bytes(batch, heads, splits):
    """Bytes of workspace attention_decode_int4kv_split needs (its partials, fp32)."""
    n = ctypes.c_int64(0)
    _check("rbq_attention_split_workspace_bytes",
           lib().rbq_attention_split_workspace_bytes(int(batch), int(heads), int(splits), ctypes.byref(n)))
    return n.value


def attention_decode_int4kv_split(q, k_codes, k_scales, v_codes, v_scales, softmax_scale, splits, *, seq=None,
                                  out=None, workspace=None, stream=None):
    """attention_decode_int4kv with each (batch, head)'s first ``seq`` tokens cut into
    ``splits`` ranges (one workgroup each) whose partials are combined by a second kernel.
    ``workspace`` is a GPU tensor of at least attention_split_workspace_bytes(B, H, splits)
    bytes (allocated here when omitted). Returns out [B, H, 128] in q's dtype."""
    torch = _torch()
    (B, H, Hkv, seq, S_cap, D), out = _attention_operands(q, k_codes, k_scales, v_codes, v_scales, seq, out)
    need = attention_split_workspace_bytes(B, H, splits)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    _require_cuda(workspace)
    if not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous tensor on q's device")
    have = workspace.numel() * workspace.element_size()
    st = lib().attention_decode_int4kv_split(_ptr(q), _dtype_code(q.dtype), _ptr(k_codes), _ptr(k_scales),
                                             _ptr(v_codes), _ptr(v_scales), _dtype_code(k_scales.dtype), B, H, Hkv,
                                             seq, S_cap, D, float(softmax_scale), int(splits), _ptr(workspace), have,
                                             _ptr(out), _stream(stream, q.device))
    _check("attention_decode_int4kv_split", st)
    return out


NOALLOC_PARTIAL_BYTES = 8 << 20  # the library's fixed partials array per GPU


def attention_decode_int4kv_split_noalloc(q, k_codes, k_scales, v_codes, v_scales, softmax_scale, splits, *,
                                          seq=None, out, stream=None):
    """attention_decode_int4kv_split with the partials in the library's fixed device array
    (8 MiB per GPU: batch * heads * splits * 520 bytes at most): nothing is allocated, so
    ``out`` [B, H, 128] in q's dtype must be passed. Calls that overlap on one GPU race."""
    if out is None:
        raise ValueError("attention_decode_int4kv_split_noalloc allocates nothing: pass out")
    if q.dim() == 3 and q.shape[0] * q.shape[1] * int(splits) * 520 > NOALLOC_PARTIAL_BYTES:
        raise ValueError(f"attention_decode_int4kv_split_noalloc: batch * heads * splits * 520 bytes of partials "
                         f"exceed the library's fixed {NOALLOC_PARTIAL_BYTES} bytes")
    (B, H, Hkv, seq, S_cap, D), out = _attention_operands(q, k_codes, k_scales, v_codes, v_scales, seq, out)
    st = lib().attention_decode_int4kv_split_noalloc(_ptr(q), _dtype_code(q.dtype), _ptr(k_codes), _ptr(k_scales),
                                                     _ptr(v_codes), _ptr(v_scales), _dtype_code(k_scales.dtype), B,
                                                     H, Hkv, seq, S_cap, D, float(softmax_scale), int(splits),
                                                     _ptr(out), _stream(stream, q.device))
    _check("attention_decode_int4kv_split_noalloc", st)
    return out


def hbm_probe(src, read_bytes_per_block, dst, write_bytes_per_block, blocks, *, stream=None):
    """Measurement only: the streaming probe of the C ABI (rbq_hbm_probe). ``src`` and
    ``dst`` are GPU tensors of at least blocks * read / write bytes per block (``dst`` at
    least 16 * blocks bytes when nothing is written per block)."""
    _require_cuda(src, dst)
    need_src = int(blocks) * int(read_bytes_per_block)
    need_dst = int(blocks) * (int(write_bytes_per_block) if write_bytes_per_block else 16)
    if src.numel() * src.element_size() < need_src or dst.numel() * dst.element_size() < need_dst:
        raise ValueError("probe buffers are smaller than the blocks would touch")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("probe buffers must be contiguous")
    st = lib().rbq_hbm_probe(_ptr(src), int(read_bytes_per_block), _ptr(dst), int(write_bytes_per_block),
                             int(blocks), _stream(stream, dst.device))
    _check("rbq_hbm_probe", st)
