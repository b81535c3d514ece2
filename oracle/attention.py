"""Decode attention over an INT4 key/value cache, in float64.

Test infrastructure (see the package docstring): not part of the product path.

Sources (restated): "SpinQuant, when rotations are worth learning", section "Four rotation
sites": R3 is a fixed Hadamard rotation applied to queries and keys after RoPE so that the
KV cache can be quantized; because the rotation is orthogonal, q . k is unchanged when
both are rotated, so attention scores can be taken between the rotated query and the
dequantized rotated keys. The values are cached in their own (R2-rotated) basis,
quantized per (token, head) with the same absmax INT4 quantizer ("SpinQuant Guide:
Learned Rotations for 4-Bit LLMs", step-size equation).

For one query position of head h (key/value head kvh = h // (H / Hkv)):
    score[s] = softmax_scale * sum_d q[d] * k_scale[s] * k_code[s, d]
    p = softmax(score) over s (subtracting the maximum first)
    out[d] = sum_s p[s] * v_scale[s] * v_code[s, d]
"""

import numpy as np


def attention_decode(q, k_codes, k_scales, v_codes, v_scales, softmax_scale):
    """q [B, H, D]; k_codes, v_codes int codes [B, Hkv, S, D]; k_scales, v_scales [B, Hkv, S]
    (stored scale values); H a multiple of Hkv. Returns (out [B, H, D], p [B, H, S]) in
    float64."""
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_codes, dtype=np.float64)
    vc = np.asarray(v_codes, dtype=np.float64)
    ks = np.asarray(k_scales, dtype=np.float64)
    vs = np.asarray(v_scales, dtype=np.float64)
    B, H, D = q.shape
    Hkv = kc.shape[1]
    if H % Hkv:
        raise ValueError("the number of query heads must be a multiple of the key/value heads")
    group = H // Hkv
    k = kc * ks[..., None]                      # dequantized keys [B, Hkv, S, D]
    v = vc * vs[..., None]
    k_h = np.repeat(k, group, axis=1)           # [B, H, S, D]
    v_h = np.repeat(v, group, axis=1)
    score = np.einsum("bhd,bhsd->bhs", q, k_h) * softmax_scale
    score = score - score.max(axis=-1, keepdims=True)
    e = np.exp(score)
    p = e / e.sum(axis=-1, keepdims=True)
    out = np.einsum("bhs,bhsd->bhd", p, v_h)
    return out, p
