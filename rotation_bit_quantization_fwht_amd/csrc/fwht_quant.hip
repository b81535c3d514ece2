// HIP kernels and C-ABI entry points for the fused Hadamard rotation + INT4 quantizer:
// hadamard_quant_int4 (rows of any length 2..32768; the R4 down-projection path and
// offline weight rotation) and kv_rotate_quant (R3 on post-RoPE Q and K per head).
// The workgroup body lives in fwht_engine.h, the gfx950 context in devctx.h and the
// kernel instantiations (one translation unit per row length) in fwht_kernels.hip; this
// file validates arguments, fills the kernel arguments and dispatches on log2 n.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "../../include/rbq.h"
#include "fwht_engine.h"
#include "validate.h"
#include "diag.h"

namespace rbq {

template <int K>
hipError_t fwht_launch(const KArgs& a, int in, bool rot, bool fourd, bool fast, bool rope, bool cache,
                       hipStream_t s);

static hipError_t dispatch(int k, const KArgs& a, int in, bool rot, bool fourd, bool fast, bool rope,
                           hipStream_t s, bool cache = false) {
  switch (k) {
    case 1: return fwht_launch<1>(a, in, rot, fourd, fast, rope, cache, s);
    case 2: return fwht_launch<2>(a, in, rot, fourd, fast, rope, cache, s);
    case 3: return fwht_launch<3>(a, in, rot, fourd, fast, rope, cache, s);
    case 4: return fwht_launch<4>(a, in, rot, fourd, fast, rope, cache, s);
    case 5: return fwht_launch<5>(a, in, rot, fourd, fast, rope, cache, s);
    case 6: return fwht_launch<6>(a, in, rot, fourd, fast, rope, cache, s);
    case 7: return fwht_launch<7>(a, in, rot, fourd, fast, rope, cache, s);
    case 8: return fwht_launch<8>(a, in, rot, fourd, fast, rope, cache, s);
    case 9: return fwht_launch<9>(a, in, rot, fourd, fast, rope, cache, s);
    case 10: return fwht_launch<10>(a, in, rot, fourd, fast, rope, cache, s);
    case 11: return fwht_launch<11>(a, in, rot, fourd, fast, rope, cache, s);
    case 12: return fwht_launch<12>(a, in, rot, fourd, fast, rope, cache, s);
    case 13: return fwht_launch<13>(a, in, rot, fourd, fast, rope, cache, s);
    case 14: return fwht_launch<14>(a, in, rot, fourd, fast, rope, cache, s);
    case 15: return fwht_launch<15>(a, in, rot, fourd, fast, rope, cache, s);
  }
  return hipErrorInvalidValue;
}

// rows per workgroup (log2) of the plan a launch will use
static int rows_log(int k, int in, bool rot) { return make_plan(k, use_matrix_plan(k, in, rot)).r; }
// log2 of the waves of a kernel's workgroup (its threads are 64 << this)
static int threads_log(int k, int in, bool rot) { return make_plan(k, use_matrix_plan(k, in, rot)).w; }

static int in_kind(rbq_dtype d) { return d == RBQ_F32 ? IN_F32 : (d == RBQ_BF16 ? IN_BF16 : IN_F16); }

}  // namespace rbq

using namespace rbq;

static rbq_status hq_launch(const void* x, rbq_dtype x_dtype, int64_t n, int64_t tokens,
                            int64_t x_row_stride, const void* signs, void* codes, void* scales,
                            rbq_dtype scale_dtype, float* rotated, unsigned flags,
                            hipStream_t stream, bool int8 = false) {
  const HqCheck chk = check_hadamard_quant(x, x_dtype, n, tokens, x_row_stride, codes, scales,
                                           scale_dtype, rotated, flags);
  if (chk.status != RBQ_OK || tokens == 0) return chk.status;
  const bool rot = (flags & RBQ_NO_ROTATE) == 0;
  const int rl = rows_log(chk.k, in_kind(x_dtype), rot);
  const int64_t blocks = (tokens + (int64_t{1} << rl) - 1) >> rl;
  if (blocks > 0x7FFFFFFF) return RBQ_EINVAL;
  // rows of one block are addressed with 32-bit offsets from the block's first row
  if (rl > 0 && (x_row_stride * dtype_size(x_dtype) << rl) >= (int64_t{1} << 31)) return RBQ_ENOTSUP;
  KArgs a{};
  TensorArgs& t = a.t[0];
  t.x = x;
  t.row_stride = x_row_stride;
  t.codes = codes;
  t.scales = scales;
  t.rot32 = rotated;
  t.signs = signs;
  t.mode = MODE_QUANT | (rotated ? MODE_ROT32 : 0u);
  t.rows = tokens;
  a.t[1] = t;
  a.blocks0 = (uint32_t)blocks;
  a.nblocks = (uint32_t)blocks;
  a.opts = ((flags & RBQ_PACKED) ? OPT_PACKED : 0u) | (scale_dtype == RBQ_F16 ? OPT_SCALE_F16 : 0u) |
           (int8 ? OPT_INT8 : 0u);
  const bool fast = (flags & RBQ_PACKED) && rotated == nullptr;
  if (diag_log())
    fprintf(stderr, "rbq: hadamard_quant n=%lld tokens=%lld dtype=%d rotate=%d signs=%d int8=%d packed=%d "
            "fast=%d blocks=%lld\n", (long long)n, (long long)tokens, (int)x_dtype, (int)rot, signs != nullptr,
            (int)int8, (flags & RBQ_PACKED) != 0, (int)fast, (long long)blocks);
  if (diag_fail_launch()) return RBQ_EHIP;
  if (dispatch(chk.k, a, in_kind(x_dtype), rot, false, fast, false, stream) != hipSuccess)
    return RBQ_EHIP;
  return RBQ_OK;
}

extern "C" rbq_status hadamard_quant_int4(const void* x, rbq_dtype x_dtype, int64_t n,
                                          int64_t tokens, int64_t x_row_stride, void* codes,
                                          void* scales, rbq_dtype scale_dtype, float* rotated,
                                          unsigned flags, hipStream_t stream) {
  return hq_launch(x, x_dtype, n, tokens, x_row_stride, nullptr, codes, scales, scale_dtype,
                   rotated, flags, stream);
}

extern "C" rbq_status hadamard_quant_int4_signed(const void* x, rbq_dtype x_dtype, int64_t n,
                                                 int64_t tokens, int64_t x_row_stride,
                                                 const void* signs, void* codes, void* scales,
                                                 rbq_dtype scale_dtype, float* rotated,
                                                 unsigned flags, hipStream_t stream) {
  const rbq_status st = check_signs(x_dtype, n, tokens, signs, flags);
  if (st != RBQ_OK) return st;
  return hq_launch(x, x_dtype, n, tokens, x_row_stride, signs, codes, scales, scale_dtype,
                   rotated, flags, stream);
}

extern "C" rbq_status hadamard_quant_int8(const void* x, rbq_dtype x_dtype, int64_t n,
                                          int64_t tokens, int64_t x_row_stride, int8_t* codes,
                                          void* scales, rbq_dtype scale_dtype, float* rotated,
                                          unsigned flags, hipStream_t stream) {
  if (flags & RBQ_PACKED) return RBQ_EINVAL;  // one code per byte
  return hq_launch(x, x_dtype, n, tokens, x_row_stride, nullptr, codes, scales, scale_dtype,
                   rotated, flags, stream, true);
}

static rbq_status kv_launch(const void* q, const void* k, rbq_dtype dtype, int64_t batch,
                            int64_t heads, int64_t seq, int64_t head_dim,
                            const int64_t q_strides[4], const int64_t k_strides[4],
                            const float* rope_cos, const float* rope_sin, int64_t rope_pos0,
                            uint8_t* q_codes, void* q_scales, uint8_t* k_codes, void* k_scales,
                            rbq_dtype scale_dtype, void* q_rotated, unsigned flags,
                            hipStream_t stream) {
  const KvCheck chk = check_kv(q, k, dtype, batch, heads, seq, head_dim, q_strides, k_strides,
                               q_codes, q_scales, k_codes, k_scales, scale_dtype, q_rotated, flags);
  if (chk.status != RBQ_OK) return chk.status;
  if (batch == 0 || heads == 0 || seq == 0) return RBQ_OK;
  if (!chk.flat && (chk.k < 6 || chk.k > 8)) return RBQ_ENOTSUP;  // strided only for d in {64,128,256}
  const int64_t rows = batch * heads * seq;
  const int rl = rows_log(chk.k, in_kind(dtype), true);
  const int64_t blocks = (rows + (int64_t{1} << rl) - 1) >> rl;
  if (chk.flat && (std::max(chk.q_rs, chk.k_rs) * 2 << rl) >= (int64_t{1} << 31)) return RBQ_ENOTSUP;
  if (2 * blocks > 0x7FFFFFFF) return RBQ_EINVAL;
  KArgs a{};
  const bool rot_only = (flags & RBQ_Q_ROTATE_ONLY) != 0;
  const void* src[2] = {q, k};
  const int64_t* st[2] = {q_strides, k_strides};
  const int64_t rs[2] = {chk.q_rs, chk.k_rs};
  for (int i = 0; i < 2; ++i) {
    TensorArgs& t = a.t[i];
    t.x = src[i];
    t.row_stride = rs[i];
    t.sb = st[i][0];
    t.sh = st[i][1];
    t.ss = st[i][2];
    t.seq = (uint32_t)seq;
    t.heads = (uint32_t)heads;
    t.div_s = make_fastdiv((uint32_t)seq);
    t.div_h = make_fastdiv((uint32_t)heads);
    t.rope_cos = rope_cos;
    t.rope_sin = rope_sin;
    t.rope_pos0 = (uint32_t)rope_pos0;
    t.rows = rows;
    if (rope_cos) set_rope_order_rt(t, chk.k);
  }
  a.t[0].codes = q_codes;
  a.t[0].scales = q_scales;
  a.t[0].rot16 = (uint16_t*)q_rotated;
  a.t[0].mode = rot_only ? MODE_ROT16 : MODE_QUANT;
  a.t[1].codes = k_codes;
  a.t[1].scales = k_scales;
  a.t[1].mode = MODE_QUANT;
  a.blocks0 = (uint32_t)blocks;
  a.nblocks = (uint32_t)(2 * blocks);
  a.opts = OPT_PACKED | (scale_dtype == RBQ_F16 ? OPT_SCALE_F16 : 0u);
  if (diag_log())
    fprintf(stderr, "rbq: kv_rotate_quant B=%lld H=%lld S=%lld D=%lld dtype=%d flat=%d rope=%d q_rotate_only=%d "
            "blocks=%lld\n", (long long)batch, (long long)heads, (long long)seq, (long long)head_dim, (int)dtype,
            (int)chk.flat, rope_cos != nullptr, (int)rot_only, (long long)(2 * blocks));
  if (diag_fail_launch()) return RBQ_EHIP;
  if (dispatch(chk.k, a, in_kind(dtype), true, !chk.flat, !rot_only, rope_cos != nullptr, stream) !=
      hipSuccess)
    return RBQ_EHIP;
  return RBQ_OK;
}

extern "C" rbq_status kv_rotate_quant(const void* q, const void* k, rbq_dtype dtype, int64_t batch,
                                      int64_t heads, int64_t seq, int64_t head_dim,
                                      const int64_t q_strides[4], const int64_t k_strides[4],
                                      uint8_t* q_codes, void* q_scales, uint8_t* k_codes,
                                      void* k_scales, rbq_dtype scale_dtype, void* q_rotated,
                                      unsigned flags, hipStream_t stream) {
  return kv_launch(q, k, dtype, batch, heads, seq, head_dim, q_strides, k_strides, nullptr,
                   nullptr, 0, q_codes, q_scales, k_codes, k_scales, scale_dtype, q_rotated,
                   flags, stream);
}

extern "C" rbq_status kv_rope_rotate_quant(const void* q, const void* k, rbq_dtype dtype,
                                           int64_t batch, int64_t heads, int64_t seq,
                                           int64_t head_dim, const int64_t q_strides[4],
                                           const int64_t k_strides[4], const float* rope_cos,
                                           const float* rope_sin, int64_t rope_positions,
                                           int64_t rope_pos0, uint8_t* q_codes, void* q_scales,
                                           uint8_t* k_codes, void* k_scales,
                                           rbq_dtype scale_dtype, void* q_rotated,
                                           unsigned flags, hipStream_t stream) {
  const rbq_status st = check_rope(dtype, batch, heads, seq, head_dim, rope_cos, rope_sin,
                                   rope_positions, rope_pos0);
  if (st != RBQ_OK) return st;
  return kv_launch(q, k, dtype, batch, heads, seq, head_dim, q_strides, k_strides, rope_cos,
                   rope_sin, rope_pos0, q_codes, q_scales, k_codes, k_scales, scale_dtype,
                   q_rotated, flags, stream);
}


// ------------------------------------------------------------------ KV4 cache append

namespace rbq {

// the (batch, head, token) addressing of one [B, heads, S, D] tensor
static void set_bhs(TensorArgs& t, const void* x, int64_t heads, int64_t seq, const int64_t st[4]) {
  t.x = x;
  t.row_stride = st[2];
  t.sb = st[0];
  t.sh = st[1];
  t.ss = st[2];
  t.seq = (uint32_t)seq;
  t.heads = (uint32_t)heads;
  t.div_s = make_fastdiv((uint32_t)seq);
  t.div_h = make_fastdiv((uint32_t)heads);
}

}  // namespace rbq

extern "C" rbq_status kv_cache_append_int4(const void* q, const void* k, const void* v, rbq_dtype dtype,
                                           int64_t batch, int64_t heads, int64_t kv_heads, int64_t seq,
                                           int64_t head_dim, const int64_t q_strides[4],
                                           const int64_t k_strides[4], const int64_t v_strides[4],
                                           const float* rope_cos, const float* rope_sin,
                                           int64_t rope_positions, int64_t pos0, int64_t seq_cap,
                                           void* q_rotated, uint8_t* k_cache, void* k_cache_scales,
                                           uint8_t* v_cache, void* v_cache_scales,
                                           rbq_dtype scale_dtype, hipStream_t stream) {
  const CacheCheck chk = check_cache_append(q, k, v, dtype, batch, heads, kv_heads, seq, head_dim, q_strides,
                                            k_strides, v_strides, rope_cos, rope_sin, rope_positions, pos0,
                                            seq_cap, q_rotated, k_cache, k_cache_scales, v_cache,
                                            v_cache_scales, scale_dtype);
  if (chk.status != RBQ_OK || batch == 0 || kv_heads == 0 || seq == 0) return chk.status;
  const bool rope = rope_cos != nullptr;
  const int in = in_kind(dtype);
  const int rl = rows_log(chk.k, in, true);
  const int64_t rows_q = q ? batch * heads * seq : 0, rows_kv = batch * kv_heads * seq;
  const int64_t bq = (rows_q + (int64_t{1} << rl) - 1) >> rl, bk = (rows_kv + (int64_t{1} << rl) - 1) >> rl;
  const int64_t ssz = dtype_size(scale_dtype), half = head_dim / 2;
  // launch 1: Q (RoPE, rotation, 16-bit output) and K (RoPE, rotation, INT4 into the cache)
  KArgs a{};
  TensorArgs& tq = a.t[0];
  TensorArgs& tk = a.t[1];
  if (q) {
    set_bhs(tq, q, heads, seq, q_strides);
    tq.rot16 = (uint16_t*)q_rotated;
    tq.mode = MODE_ROT16;
    tq.rows = rows_q;
  }
  set_bhs(tk, k, kv_heads, seq, k_strides);
  tk.codes = k_cache + pos0 * half;
  tk.scales = (char*)k_cache_scales + pos0 * ssz;
  tk.mode = MODE_QUANT;
  tk.rows = rows_kv;
  tk.out_cap = (uint32_t)seq_cap;
  for (TensorArgs* t : {&tq, &tk}) {
    t->rope_cos = rope_cos;
    t->rope_sin = rope_sin;
    t->rope_pos0 = (uint32_t)pos0;
    if (rope_cos) set_rope_order_rt(*t, chk.k);
  }
  // V (INT4 without rotation into the cache) in the same launch: the blocks after Q's and
  // K's take n / 8 lanes per row (as_is_rows)
  const int64_t vrows_per_block = (int64_t{64} << threads_log(chk.k, in, true)) / (head_dim / 8);
  const int64_t bv = (rows_kv + vrows_per_block - 1) / vrows_per_block;
  if (bq + bk + bv > 0x7FFFFFFF) return RBQ_EINVAL;
  TensorArgs& tv = a.tv;
  set_bhs(tv, v, kv_heads, seq, v_strides);
  tv.codes = v_cache + pos0 * half;
  tv.scales = (char*)v_cache_scales + pos0 * ssz;
  tv.mode = MODE_QUANT;
  tv.rows = rows_kv;
  tv.out_cap = (uint32_t)seq_cap;
  a.blocks0 = (uint32_t)bq;
  a.blocks1 = (uint32_t)(bq + bk);
  a.nblocks = (uint32_t)(bq + bk + bv);
  a.opts = OPT_PACKED | (scale_dtype == RBQ_F16 ? OPT_SCALE_F16 : 0u);
  if (diag_log())
    fprintf(stderr, "rbq: kv_cache_append B=%lld H=%lld Hkv=%lld S=%lld D=%lld pos0=%lld cap=%lld rope=%d q=%d "
            "blocks=%lld+%lld\n", (long long)batch, (long long)heads, (long long)kv_heads, (long long)seq,
            (long long)head_dim, (long long)pos0, (long long)seq_cap, (int)rope, q != nullptr,
            (long long)(bq + bk), (long long)bv);
  if (diag_fail_launch()) return RBQ_EHIP;
  if (dispatch(chk.k, a, in, true, true, false, rope, stream, true) != hipSuccess) return RBQ_EHIP;
  return RBQ_OK;
}
