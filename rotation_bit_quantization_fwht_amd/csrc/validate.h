// Host-side argument checks shared by the C-ABI entry points. Pure C++: no HIP call is
// made before these succeed, so invalid calls are rejected even without a GPU.
#pragma once

#include <stdint.h>

#include "../../include/rbq.h"

namespace rbq {

inline bool is_pow2(int64_t n) { return n > 0 && (n & (n - 1)) == 0; }

inline int ilog2(int64_t n) {
  int k = 0;
  while ((int64_t{1} << k) < n) ++k;
  return k;
}

inline bool aligned(const void* p, uint64_t a) { return ((uintptr_t)p % a) == 0; }

inline int dtype_size(rbq_dtype d) {
  switch (d) {
    case RBQ_F32: return 4;
    case RBQ_BF16: return 2;
    case RBQ_F16: return 2;
  }
  return 0;
}

inline bool valid_in_dtype(int d) { return d == RBQ_F32 || d == RBQ_BF16 || d == RBQ_F16; }
inline bool valid_scale_dtype(int d) { return d == RBQ_F32 || d == RBQ_F16; }

struct HqCheck {
  rbq_status status;
  int k;
};

inline HqCheck check_hadamard_quant(const void* x, int x_dtype, int64_t n, int64_t tokens,
                                    int64_t x_row_stride, const void* codes, const void* scales,
                                    int scale_dtype, const float* rotated, unsigned flags) {
  HqCheck r{RBQ_EINVAL, 0};
  if (flags & ~(unsigned)(RBQ_PACKED | RBQ_NO_ROTATE)) return r;
  if (!valid_in_dtype(x_dtype) || !valid_scale_dtype(scale_dtype)) return r;
  if (!is_pow2(n) || n < 2 || n > 32768) return r;
  if (tokens < 0) return r;
  r.k = ilog2(n);
  if (tokens == 0) { r.status = RBQ_OK; return r; }
  if (!x || !codes || !scales) return r;
  if (x_row_stride < n) return r;
  const int64_t esz = dtype_size((rbq_dtype)x_dtype);
  const int64_t align = (n * esz < 16) ? n * esz : 16;
  if (!aligned(x, (uint64_t)align) || ((x_row_stride * esz) % align) != 0) return r;
  if (!aligned(codes, 16)) return r;
  if (!aligned(scales, (uint64_t)dtype_size((rbq_dtype)scale_dtype))) return r;
  if (rotated && !aligned(rotated, 16)) return r;
  r.status = RBQ_OK;
  return r;
}

// the +-1 diagonal of the randomized transform: one value per element in the input dtype,
// aligned like a row; it only makes sense with the rotation
inline rbq_status check_signs(int x_dtype, int64_t n, int64_t tokens, const void* signs,
                              unsigned flags) {
  if (flags & RBQ_NO_ROTATE) return RBQ_EINVAL;
  if (tokens == 0) return RBQ_OK;
  if (!signs || !valid_in_dtype(x_dtype) || !is_pow2(n)) return RBQ_EINVAL;
  const int64_t esz = dtype_size((rbq_dtype)x_dtype);
  const int64_t align = (n * esz < 16) ? n * esz : 16;
  if (!aligned(signs, (uint64_t)align)) return RBQ_EINVAL;
  return RBQ_OK;
}

struct KvCheck {
  rbq_status status;
  int k;
  bool flat;            // rows form an arithmetic progression in both tensors
  int64_t q_rs, k_rs;   // row strides when flat
};

inline bool kv_flat_stride(int64_t B, int64_t H, int64_t S, int64_t D, const int64_t st[4],
                           int64_t* rs) {
  int64_t c;
  if (S > 1) c = st[2];
  else if (H > 1) c = st[1];
  else if (B > 1) c = st[0];
  else c = D;
  if (S > 1 && st[2] != c) return false;
  if (H > 1 && st[1] != S * c) return false;
  if (B > 1 && st[0] != H * S * c) return false;
  *rs = c;
  return true;
}

inline KvCheck check_kv(const void* q, const void* k, int dtype, int64_t B, int64_t H, int64_t S,
                        int64_t D, const int64_t* qs, const int64_t* ks, const void* q_codes,
                        const void* q_scales, const void* k_codes, const void* k_scales,
                        int scale_dtype, const void* q_rot, unsigned flags) {
  KvCheck r{RBQ_EINVAL, 0, false, 0, 0};
  if (flags & ~(unsigned)RBQ_Q_ROTATE_ONLY) return r;
  if (dtype != RBQ_BF16 && dtype != RBQ_F16) return r;
  if (!valid_scale_dtype(scale_dtype)) return r;
  if (B < 0 || H < 0 || S < 0) return r;
  if (!is_pow2(D) || D < 8 || D > 32768) return r;
  r.k = ilog2(D);
  if (B == 0 || H == 0 || S == 0) { r.status = RBQ_OK; return r; }
  if (!q || !k || !qs || !ks) return r;
  if (B * H > (int64_t{1} << 31) || B * H * S >= (int64_t{1} << 31)) return r;
  const bool rot_only = (flags & RBQ_Q_ROTATE_ONLY) != 0;
  if (rot_only) {
    if (!q_rot || !aligned(q_rot, 16)) return r;
  } else {
    if (!q_codes || !q_scales || !aligned(q_codes, 16)) return r;
    if (!aligned(q_scales, (uint64_t)dtype_size((rbq_dtype)scale_dtype))) return r;
  }
  if (!k_codes || !k_scales || !aligned(k_codes, 16)) return r;
  if (!aligned(k_scales, (uint64_t)dtype_size((rbq_dtype)scale_dtype))) return r;
  for (const int64_t* st : {qs, ks}) {
    if (st[3] != 1) return r;
    for (int i = 0; i < 3; ++i)
      if (st[i] < 0 || (st[i] * 2) % 16 != 0) return r;
  }
  if (!aligned(q, 16) || !aligned(k, 16)) return r;
  r.flat = kv_flat_stride(B, H, S, D, qs, &r.q_rs) && kv_flat_stride(B, H, S, D, ks, &r.k_rs);
  r.status = RBQ_OK;
  return r;
}

// RoPE tables: fp32 [rope_positions, head_dim / 2], 16-byte aligned, covering positions
// rope_pos0 .. rope_pos0 + seq - 1; head_dim 64, 128 or 256 (the layouts that hold each
// load's partner elements and table values)
inline rbq_status check_rope(int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                             const float* cos, const float* sin, int64_t positions,
                             int64_t pos0) {
  if (B < 0 || H < 0 || S < 0 || pos0 < 0 || positions < 0) return RBQ_EINVAL;
  if (B == 0 || H == 0 || S == 0) return RBQ_OK;
  if (!cos || !sin || !aligned(cos, 16) || !aligned(sin, 16)) return RBQ_EINVAL;
  if (pos0 + S > positions || positions > (int64_t{1} << 30)) return RBQ_EINVAL;
  if (dtype != RBQ_BF16 && dtype != RBQ_F16) return RBQ_EINVAL;
  if (D != 64 && D != 128 && D != 256) return RBQ_ENOTSUP;
  return RBQ_OK;
}

struct CacheCheck {
  rbq_status status;
  int k;  // log2 head_dim
};

// kv_cache_append_int4: [B, heads, S, D] Q (optional), [B, kv_heads, S, D] K and V with any
// element strides (d stride 1, 16-byte aligned vectors); caches [B, kv_heads, seq_cap, D/2]
// and [B, kv_heads, seq_cap] receiving positions pos0 .. pos0 + S - 1
inline CacheCheck check_cache_append(const void* q, const void* k, const void* v, int dtype, int64_t B,
                                     int64_t H, int64_t Hkv, int64_t S, int64_t D, const int64_t* qs,
                                     const int64_t* ks, const int64_t* vs, const float* cos,
                                     const float* sin, int64_t positions, int64_t pos0, int64_t cap,
                                     const void* q_rot, const void* kc, const void* ksc, const void* vc,
                                     const void* vsc, int scale_dtype) {
  CacheCheck r{RBQ_EINVAL, 0};
  if (dtype != RBQ_BF16 && dtype != RBQ_F16) return r;
  if (!valid_scale_dtype(scale_dtype)) return r;
  if (B < 0 || H < 0 || Hkv < 0 || S < 0 || pos0 < 0 || cap < 0) return r;
  if (pos0 + S > cap) return r;
  if (Hkv > 0 && H % Hkv != 0) return r;
  if ((cos == nullptr) != (sin == nullptr)) return r;
  if (D != 64 && D != 128 && D != 256) {
    r.status = (is_pow2(D) && D >= 8 && D <= 32768) ? RBQ_ENOTSUP : RBQ_EINVAL;
    return r;
  }
  r.k = ilog2(D);
  if (B == 0 || Hkv == 0 || S == 0) { r.status = RBQ_OK; return r; }
  if (B * H > (int64_t{1} << 31) || B * H * S >= (int64_t{1} << 31) || B * Hkv * cap >= (int64_t{1} << 31))
    return r;
  if (cos) {
    const rbq_status rs = check_rope(dtype, B, Hkv, S, D, cos, sin, positions, pos0);
    if (rs != RBQ_OK) { r.status = rs; return r; }
  }
  if ((q == nullptr) != (q_rot == nullptr)) return r;
  if (q && (!qs || !aligned(q, 16) || !aligned(q_rot, 16))) return r;
  if (!k || !v || !ks || !vs || !aligned(k, 16) || !aligned(v, 16)) return r;
  if (!kc || !vc || !ksc || !vsc || !aligned(kc, 16) || !aligned(vc, 16)) return r;
  const uint64_t ssz = (uint64_t)dtype_size((rbq_dtype)scale_dtype);
  if (!aligned(ksc, ssz) || !aligned(vsc, ssz)) return r;
  for (const int64_t* st : {qs, ks, vs}) {
    if (!st) continue;
    if (st[3] != 1) return r;
    for (int i = 0; i < 3; ++i)
      if (st[i] < 0 || (st[i] * 2) % 16 != 0) return r;
  }
  r.status = RBQ_OK;
  return r;
}

inline rbq_status check_gemm(const void* qA, const void* sA, const void* qW, const void* sW,
                             int scale_dtype, int64_t M, int64_t N, int64_t K, const void* out,
                             const void* acc) {
  if (!valid_scale_dtype(scale_dtype)) return RBQ_EINVAL;
  if (M < 0 || N < 0 || K <= 0 || (K & 1)) return RBQ_EINVAL;
  if (M == 0 || N == 0) return RBQ_OK;
  if (!qA || !sA || !qW || !sW || !out) return RBQ_EINVAL;
  if (!aligned(qA, 16) || !aligned(qW, 16) || !aligned(out, 16)) return RBQ_EINVAL;
  if (acc && !aligned(acc, 16)) return RBQ_EINVAL;
  const uint64_t ssz = (uint64_t)dtype_size((rbq_dtype)scale_dtype);
  if (!aligned(sA, ssz) || !aligned(sW, ssz)) return RBQ_EINVAL;
  if (K % 128 != 0 || K > 65536 || N % 8 != 0) return RBQ_ENOTSUP;
  if (M > (int64_t{1} << 30) || N > (int64_t{1} << 30)) return RBQ_ENOTSUP;
  return RBQ_OK;
}

}  // namespace rbq
