// Decode attention over the INT4 key/value cache that kv_rotate_quant (keys, R3-rotated)
// and hadamard_quant_int4 without rotation (values) write: one query position per
// (batch, head), head_dim 128, grouped key/value heads.
//
//   score[s] = softmax_scale * sum_d q[d] * k_scale[s] * k_code[s, d]
//   out[d]   = sum_s softmax(score)[s] * v_scale[s] * v_code[s, d]
//
// The query is the rotated one (the R3 rotation of the keys applied to it too), so the
// scores equal those of the unrotated pair ("SpinQuant, when rotations are worth
// learning", section "Four rotation sites": R3 is there so that K can be cached in INT4).
//
// One 512-thread workgroup per (batch, head), one pass over the cache. Sixteen lanes share
// one cached token: lane c takes dims 8c .. 8c + 7, i.e. one dword of codes of the token's
// 64-byte row, so a wave reads four consecutive rows (256 contiguous bytes) per load. Each
// 16-lane group runs its own online softmax over its tokens (every 32nd token): per batch
// of kAttnU tokens it takes the scores, raises its running maximum, rescales its sum and
// output, and accumulates the value rows with the probabilities. At the end the 32
// groups' (maximum, sum, output) triples are merged in LDS.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/rbq.h"
#include "common.h"
#include "diag.h"
#include "validate.h"

namespace rbq {

struct AttnArgs {
  float* part;          // split kernel: [B * H, splits, 2 + 128] partial (max, sum, output)
  int splits, chunk;    // split kernel: token ranges [sp * chunk, (sp + 1) * chunk)
  const void* q;        // [B, H, 128] bf16 or fp16
  const uint8_t* kc;    // [B, Hkv, S_cap, 64]
  const void* ks;       // [B, Hkv, S_cap]
  const uint8_t* vc;
  const void* vs;
  void* out;            // [B, H, 128], the query's format
  int H, Hkv, S, S_cap;
  float scale;
  int q_f16, scale_f16;
};

constexpr int kAttnThreads = 512;  // (256: 48 us, 1024: 40 us on the [16, 32, 2048, 128] cache)
constexpr int kAttnGroups = kAttnThreads / 16;  // token groups of sixteen lanes
constexpr int kAttnD = 128;
constexpr int kAttnU = 8;  // tokens per group and batch

__device__ __forceinline__ float attn_load16(const void* p, int64_t i, int f16) {
  const uint32_t h = ((const uint16_t*)p)[i];
  return f16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)h) : bits_f32(h << 16);
}

// the eight codes of a dword of packed codes (low nibble first), each as 16 x code: the
// even codes shifted into the high nibbles of the bytes and the odd codes masked in place
// make signed bytes, which convert one per instruction (sign-extending byte selects); the
// factor 16 is taken out of the other operand exactly (a power of two)
__device__ __forceinline__ void attn_codes16(uint32_t w, float (&c)[8]) {
  const uint32_t ev = (w << 4) & 0xF0F0F0F0u, od = w & 0xF0F0F0F0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[2 * j] = (float)(int8_t)(ev >> (8 * j));
    c[2 * j + 1] = (float)(int8_t)(od >> (8 * j));
  }
}

// the value of another lane of the same 16-lane row, by a DPP move (CTRL: the DPP
// control word)
template <int CTRL>
__device__ __forceinline__ float attn_dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// sum over each row of sixteen lanes, the same bits on every lane of the row: four DPP
// steps (pairs, quads, the two quads of each half, the two halves), each adding the values
// of two lanes that then hold the same sum in swapped order. A row is one token group, so
// its lanes are active or inactive together.
__device__ __forceinline__ float attn_row16_sum(float v) {
  v += attn_dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += attn_dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += attn_dpp<0x141>(v);  // row_half_mirror
  v += attn_dpp<0x140>(v);  // row_mirror
  return v;
}

// one batch of a group's tokens: the lane's dword of each key and value row and the
// tokens' scales. The loads are buffer loads range-checked against the head's first S
// tokens: a token past the sequence reads zeros (its score is then set to -inf, so it
// weighs 0), and no load is predicated.
struct AttnBatch {
  uint32_t kw[kAttnU], vw[kAttnU];
  float ks[kAttnU], vs[kAttnU];
};

struct AttnRsrc {
  __amdgpu_buffer_rsrc_t kc, vc, ks, vs;
};

constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit data, no swizzle, range-checked

__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

template <int SF16>
__device__ __forceinline__ void attn_fetch(AttnBatch& r, const AttnRsrc& rs, int t0, int c) {
#pragma unroll
  for (int u = 0; u < kAttnU; ++u) {
    const uint32_t t = (uint32_t)(t0 + u * kAttnGroups);
    r.kw[u] = __builtin_amdgcn_raw_buffer_load_b32(rs.kc, t * 64u + 4u * c, 0, 0);
    r.vw[u] = __builtin_amdgcn_raw_buffer_load_b32(rs.vc, t * 64u + 4u * c, 0, 0);
    if constexpr (SF16) {
      r.ks[u] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs.ks, t * 2u, 0, 0));
      r.vs[u] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs.vs, t * 2u, 0, 0));
    } else {
      r.ks[u] = bits_f32(__builtin_amdgcn_raw_buffer_load_b32(rs.ks, t * 4u, 0, 0));
      r.vs[u] = bits_f32(__builtin_amdgcn_raw_buffer_load_b32(rs.vs, t * 4u, 0, 0));
    }
  }
}

// SPLIT: workgroup x takes the tokens [sp * chunk, (sp + 1) * chunk) of pair bh (x = bh *
// splits + sp) and writes its (maximum, sum, unnormalised output) to a.part instead of the
// output; attention_merge_kernel combines the splits
template <int SF16, bool SPLIT>
__global__ __launch_bounds__(kAttnThreads) void attention_decode_kernel(AttnArgs a) {
  __shared__ float part[kAttnGroups][kAttnD];
  __shared__ float gmax[kAttnGroups], gsum[kAttnGroups];
  const int bh = SPLIT ? (int)blockIdx.x / a.splits : (int)blockIdx.x;
  const int sp = SPLIT ? (int)blockIdx.x - bh * a.splits : 0;
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int tid = threadIdx.x, c = tid & 15, tg = tid >> 4;

  // the query times the softmax scale, then over 16 (exact) for the codes' factor 16
  float qd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qd[i] = (attn_load16(a.q, (int64_t)bh * kAttnD + 8 * c + i, a.q_f16) * a.scale) * 0.0625f;

  const int64_t head = (int64_t)b * a.Hkv + kvh;
  const uint32_t ssz = SF16 ? 2u : 4u;
  // this workgroup's tokens: [t_begin, t_begin + n) of the head (all S without splits)
  const int t_begin = SPLIT ? sp * a.chunk : 0;
  const int n = SPLIT ? max(0, min(a.chunk, a.S - t_begin)) : a.S;
  const int64_t tok0 = head * a.S_cap + t_begin;
  AttnRsrc rs;
  rs.kc = attn_rsrc(a.kc + tok0 * 64, (uint32_t)n * 64u);
  rs.vc = attn_rsrc(a.vc + tok0 * 64, (uint32_t)n * 64u);
  rs.ks = attn_rsrc((const char*)a.ks + tok0 * ssz, (uint32_t)n * ssz);
  rs.vs = attn_rsrc((const char*)a.vs + tok0 * ssz, (uint32_t)n * ssz);

  // the group's running maximum and sum (equal on its sixteen lanes) and its output dims
  float m_run = -INFINITY, l_run = 0.0f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;

  // per batch: scores (eight products per lane, summed over the sixteen lanes with the
  // same bits on every lane), the raised maximum, the rescaled sum
  // and output, then the value rows weighted by the probabilities. The batch's loads are
  // all issued before any is used; the other waves of the CU hide their latency. The
  // batch's first token is always in range.
  for (int t0 = tg; t0 < n; t0 += kAttnU * kAttnGroups) {
    AttnBatch r;
    attn_fetch<SF16>(r, rs, t0, c);
    float sc[kAttnU];
    float bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      float kc[8];
      attn_codes16(r.kw[u], kc);
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = fmaf(qd[i], kc[i], dot);
      dot = attn_row16_sum(dot);
      sc[u] = (t0 + u * kAttnGroups < n) ? dot * r.ks[u] : -INFINITY;
      bmax = fmaxf(bmax, sc[u]);
    }
    const float m_new = fmaxf(m_run, bmax);
    const float corr = __expf(m_run - m_new);  // 0 on the group's first batch
    l_run *= corr;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= corr;
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      const float p = __expf(sc[u] - m_new);  // 0 past the sequence
      l_run += p;
      const float pv = (p * r.vs[u]) * 0.0625f;
      float vc[8];
      attn_codes16(r.vw[u], vc);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(pv, vc[i], acc[i]);
    }
    m_run = m_new;
  }

  // ---- merge the groups: out = sum_g e^(m_g - M) acc_g / sum_g e^(m_g - M) l_g; groups
  // without tokens hold (-inf, 0, 0) and weigh 0 (group 0 always has token 0, except in
  // a split past the sequence's end, whose triple is then (-inf, 0, 0))
#pragma unroll
  for (int i = 0; i < 8; ++i) part[tg][8 * c + i] = acc[i];
  if (c == 0) {
    gmax[tg] = m_run;
    gsum[tg] = l_run;
  }
  __syncthreads();
  if (tid < kAttnD) {
    float mx = gmax[0];
#pragma unroll
    for (int g = 1; g < kAttnGroups; ++g) mx = fmaxf(mx, gmax[g]);
    float o = 0.0f, l = 0.0f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int g = 0; g < kAttnGroups; ++g) {
        const float w = __expf(gmax[g] - mx);
        o = fmaf(part[g][tid], w, o);
        l = fmaf(gsum[g], w, l);
      }
    }
    if constexpr (SPLIT) {
      float* pp = a.part + ((int64_t)bh * a.splits + sp) * (2 + kAttnD);
      pp[2 + tid] = o;
      if (tid == 0) {
        pp[0] = mx;
        pp[1] = l;
      }
      return;
    }
    o /= l;
    uint16_t bits;
    if (a.q_f16) bits = __builtin_bit_cast(uint16_t, (_Float16)o);
    else bits = (uint16_t)f32_to_bf16(o);
    ((uint16_t*)a.out)[(int64_t)bh * kAttnD + tid] = bits;
  }
}

// the splits of pair bh (one workgroup of 128 threads, one output dim each), in split
// order: out = sum_sp e^(m_sp - M) o_sp / sum_sp e^(m_sp - M) l_sp, M the largest maximum
// (split 0 always holds token 0, so M is finite); rounded to the query's format
__global__ __launch_bounds__(kAttnD) void attention_merge_kernel(AttnArgs a) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* pp = a.part + (int64_t)bh * a.splits * (2 + kAttnD);
  float mx = pp[0];
  for (int sp = 1; sp < a.splits; ++sp) mx = fmaxf(mx, pp[sp * (2 + kAttnD)]);
  float o = 0.0f, l = 0.0f;
  for (int sp = 0; sp < a.splits; ++sp) {
    const float* ps = pp + sp * (2 + kAttnD);
    const float w = __expf(ps[0] - mx);  // 0 for a split without tokens (maximum -inf)
    o = fmaf(ps[2 + d], w, o);
    l = fmaf(ps[1], w, l);
  }
  o /= l;
  uint16_t bits;
  if (a.q_f16) bits = __builtin_bit_cast(uint16_t, (_Float16)o);
  else bits = (uint16_t)f32_to_bf16(o);
  ((uint16_t*)a.out)[(int64_t)bh * kAttnD + d] = bits;
}

// checks shared by the attention entry points; RBQ_OK when a launch should follow
static rbq_status attn_check(const void* q, rbq_dtype q_dtype, const uint8_t* k_codes, const void* k_scales,
                             const uint8_t* v_codes, const void* v_scales, rbq_dtype scale_dtype, int64_t batch,
                             int64_t heads, int64_t kv_heads, int64_t seq, int64_t seq_cap, int64_t head_dim,
                             float softmax_scale, const void* out) {
  if (q_dtype != RBQ_BF16 && q_dtype != RBQ_F16) return RBQ_EINVAL;
  if (!valid_scale_dtype(scale_dtype)) return RBQ_EINVAL;
  if (batch < 0 || heads < 0 || kv_heads < 1 || seq < 1 || seq_cap < seq) return RBQ_EINVAL;
  if (heads % kv_heads != 0 || !(softmax_scale == softmax_scale)) return RBQ_EINVAL;
  if (head_dim != kAttnD) return RBQ_ENOTSUP;
  if (batch == 0 || heads == 0) return RBQ_OK;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !out) return RBQ_EINVAL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16)) return RBQ_EINVAL;
  const uint64_t ssz = (uint64_t)dtype_size(scale_dtype);
  if (!aligned(k_scales, ssz) || !aligned(v_scales, ssz)) return RBQ_EINVAL;
  // buffer offsets within one head's cache are 32-bit: seq * 64 bytes must fit
  if (batch * heads > 0x7FFFFFFF || heads > 0x7FFFFFFF || seq_cap > (int64_t{1} << 30) || seq >= (int64_t{1} << 26))
    return RBQ_ENOTSUP;
  return RBQ_OK;
}

static AttnArgs attn_args(const void* q, rbq_dtype q_dtype, const uint8_t* k_codes, const void* k_scales,
                          const uint8_t* v_codes, const void* v_scales, rbq_dtype scale_dtype, int64_t heads,
                          int64_t kv_heads, int64_t seq, int64_t seq_cap, float softmax_scale, void* out) {
  AttnArgs a{};
  a.q = q; a.kc = k_codes; a.ks = k_scales; a.vc = v_codes; a.vs = v_scales; a.out = out;
  a.H = (int)heads; a.Hkv = (int)kv_heads; a.S = (int)seq; a.S_cap = (int)seq_cap;
  a.scale = softmax_scale;
  a.q_f16 = q_dtype == RBQ_F16;
  a.scale_f16 = scale_dtype == RBQ_F16;
  return a;
}

// ---- the split partials of attention_decode_int4kv_split_noalloc: a fixed device array,
// for callers that cannot allocate (one per GPU the library runs on, held until the process
// ends). Host code never passes the array's name to a kernel (on the host it is a stand-in,
// not a device address): it uses the address hipGetSymbolAddress returns, once per device.
// Nothing in it must start at zero (the split kernel writes every partial the merge reads);
// calls that overlap on one GPU share it and race.
constexpr int64_t kAttnScratchBytes = int64_t{8} << 20;
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

constexpr int kAttnMaxDevices = 64;

// the device address of `scratch` on the current device; nullptr if it cannot be found
static float* attn_scratch_ptr() {
  static std::mutex mu;
  static float* ptrs[kAttnMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kAttnMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = (float*)p;
  }
  return ptrs[dev];
}

// bytes of split partials for batch * heads pairs and `splits` ranges
static int64_t attn_split_bytes(int64_t batch, int64_t heads, int64_t splits) {
  return batch * heads * splits * (2 + kAttnD) * (int64_t)sizeof(float);
}

// the split kernels on a workspace of at least attn_split_bytes bytes
static rbq_status attn_split_launch(AttnArgs a, int64_t batch, int64_t heads, int64_t splits, float* part,
                                    hipStream_t stream) {
  a.splits = (int)splits;
  a.chunk = (int)((a.S + splits - 1) / splits);
  a.part = part;
  const uint32_t grid = (uint32_t)(batch * heads * splits);
  if (a.scale_f16)
    hipLaunchKernelGGL((attention_decode_kernel<1, true>), dim3(grid), dim3(kAttnThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attention_decode_kernel<0, true>), dim3(grid), dim3(kAttnThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return RBQ_EHIP;
  hipLaunchKernelGGL(attention_merge_kernel, dim3((uint32_t)(batch * heads)), dim3(kAttnD), 0, stream, a);
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}

}  // namespace rbq

using namespace rbq;

extern "C" rbq_status attention_decode_int4kv(const void* q, rbq_dtype q_dtype, const uint8_t* k_codes,
                                              const void* k_scales, const uint8_t* v_codes,
                                              const void* v_scales, rbq_dtype scale_dtype, int64_t batch,
                                              int64_t heads, int64_t kv_heads, int64_t seq, int64_t seq_cap,
                                              int64_t head_dim, float softmax_scale, void* out,
                                              hipStream_t stream) {
  const rbq_status st = attn_check(q, q_dtype, k_codes, k_scales, v_codes, v_scales, scale_dtype, batch, heads,
                                   kv_heads, seq, seq_cap, head_dim, softmax_scale, out);
  if (st != RBQ_OK || batch == 0 || heads == 0) return st;
  const AttnArgs a = attn_args(q, q_dtype, k_codes, k_scales, v_codes, v_scales, scale_dtype, heads, kv_heads, seq,
                               seq_cap, softmax_scale, out);
  if (diag_log())
    fprintf(stderr, "rbq: attention_decode_int4kv B=%lld H=%lld Hkv=%lld S=%lld cap=%lld\n", (long long)batch,
            (long long)heads, (long long)kv_heads, (long long)seq, (long long)seq_cap);
  if (diag_fail_launch()) return RBQ_EHIP;
  if (a.scale_f16)
    hipLaunchKernelGGL((attention_decode_kernel<1, false>), dim3((uint32_t)(batch * heads)), dim3(kAttnThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((attention_decode_kernel<0, false>), dim3((uint32_t)(batch * heads)), dim3(kAttnThreads), 0,
                       stream, a);
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}

extern "C" rbq_status rbq_attention_split_workspace_bytes(int64_t batch, int64_t heads, int64_t splits,
                                                          int64_t* bytes) {
  if (!bytes || batch < 0 || heads < 0 || splits < 1 || splits > 4096) return RBQ_EINVAL;
  if (batch * heads > 0x7FFFFFFF) return RBQ_ENOTSUP;
  *bytes = attn_split_bytes(batch, heads, splits);
  return RBQ_OK;
}

extern "C" rbq_status attention_decode_int4kv_split(const void* q, rbq_dtype q_dtype, const uint8_t* k_codes,
                                                    const void* k_scales, const uint8_t* v_codes,
                                                    const void* v_scales, rbq_dtype scale_dtype, int64_t batch,
                                                    int64_t heads, int64_t kv_heads, int64_t seq, int64_t seq_cap,
                                                    int64_t head_dim, float softmax_scale, int64_t splits,
                                                    void* workspace, int64_t workspace_bytes, void* out,
                                                    hipStream_t stream) {
  if (splits < 1 || splits > 4096) return RBQ_EINVAL;
  const rbq_status st = attn_check(q, q_dtype, k_codes, k_scales, v_codes, v_scales, scale_dtype, batch, heads,
                                   kv_heads, seq, seq_cap, head_dim, softmax_scale, out);
  if (st != RBQ_OK || batch == 0 || heads == 0) return st;
  if (batch * heads * splits > 0x7FFFFFFF) return RBQ_ENOTSUP;
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < attn_split_bytes(batch, heads, splits))
    return RBQ_EINVAL;
  const AttnArgs a = attn_args(q, q_dtype, k_codes, k_scales, v_codes, v_scales, scale_dtype, heads, kv_heads, seq,
                               seq_cap, softmax_scale, out);
  if (diag_log())
    fprintf(stderr, "rbq: attention_decode_int4kv_split B=%lld H=%lld Hkv=%lld S=%lld cap=%lld splits=%lld\n",
            (long long)batch, (long long)heads, (long long)kv_heads, (long long)seq, (long long)seq_cap,
            (long long)splits);
  if (diag_fail_launch()) return RBQ_EHIP;
  return attn_split_launch(a, batch, heads, splits, (float*)workspace, stream);
}

extern "C" rbq_status attention_decode_int4kv_split_noalloc(const void* q, rbq_dtype q_dtype, const uint8_t* k_codes,
                                                            const void* k_scales, const uint8_t* v_codes,
                                                            const void* v_scales, rbq_dtype scale_dtype,
                                                            int64_t batch, int64_t heads, int64_t kv_heads,
                                                            int64_t seq, int64_t seq_cap, int64_t head_dim,
                                                            float softmax_scale, int64_t splits, void* out,
                                                            hipStream_t stream) {
  if (splits < 1 || splits > 4096) return RBQ_EINVAL;
  const rbq_status st = attn_check(q, q_dtype, k_codes, k_scales, v_codes, v_scales, scale_dtype, batch, heads,
                                   kv_heads, seq, seq_cap, head_dim, softmax_scale, out);
  if (st != RBQ_OK || batch == 0 || heads == 0) return st;
  if (batch * heads * splits > 0x7FFFFFFF) return RBQ_ENOTSUP;
  if (attn_split_bytes(batch, heads, splits) > kAttnScratchBytes) return RBQ_ENOTSUP;  // beyond the fixed array
  const AttnArgs a = attn_args(q, q_dtype, k_codes, k_scales, v_codes, v_scales, scale_dtype, heads, kv_heads, seq,
                               seq_cap, softmax_scale, out);
  if (diag_log())
    fprintf(stderr,
            "rbq: attention_decode_int4kv_split_noalloc B=%lld H=%lld Hkv=%lld S=%lld cap=%lld splits=%lld\n",
            (long long)batch, (long long)heads, (long long)kv_heads, (long long)seq, (long long)seq_cap,
            (long long)splits);
  if (diag_fail_launch()) return RBQ_EHIP;
  float* part = attn_scratch_ptr();
  if (!part) return RBQ_EHIP;
  return attn_split_launch(a, batch, heads, splits, part, stream);
}
