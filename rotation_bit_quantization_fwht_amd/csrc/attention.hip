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
// One 256-thread workgroup per (batch, head), or per range of its tokens in the split form,
// one pass over the cache. Four lanes share one cached token: lane c takes dims
// 32c .. 32c + 31, i.e. bytes 16c .. 16c + 15 of the token's 64-byte code row, so a wave
// reads sixteen consecutive rows (1 KiB contiguous) per 16-byte load. Each four-lane group
// runs its own online softmax over its tokens (every 64th token): per batch of kAttnU
// tokens it takes the scores, raises its running maximum, rescales its sum and output, and
// accumulates the value rows with the probabilities. At the end the 64 groups' (maximum,
// sum, output) triples are merged in LDS.
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
  int units;            // (batch, key/value head, split) triples: batch * Hkv * splits
  float scale;
  int q_f16, scale_f16;
};

constexpr int kAttnThreads = 256;
constexpr int kAttnGroups = kAttnThreads / 4;  // token groups of four lanes
constexpr int kAttnD = 128;
constexpr int kAttnU = 4;  // tokens per group and batch

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

// the value of another lane of the same quad, by a DPP move (CTRL: the DPP control word)
template <int CTRL>
__device__ __forceinline__ float attn_dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

struct AttnRsrc {
  __amdgpu_buffer_rsrc_t kc, vc, ks, vs;
};

constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit data, no swizzle, range-checked

__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

typedef uint32_t attn_u32x4 __attribute__((ext_vector_type(4)));

struct AttnBatch {
  attn_u32x4 kw[kAttnU], vw[kAttnU];
  float ks[kAttnU], vs[kAttnU];
};

template <int SF16>
__device__ __forceinline__ void attn_fetch(AttnBatch& r, const AttnRsrc& rs, int t0, int c) {
#pragma unroll
  for (int u = 0; u < kAttnU; ++u) {
    const uint32_t t = (uint32_t)(t0 + u * kAttnGroups);
    r.kw[u] = __builtin_bit_cast(attn_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.kc, t * 64u + 16u * c, 0, 0));
    r.vw[u] = __builtin_bit_cast(attn_u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs.vc, t * 64u + 16u * c, 0, 0));
    if constexpr (SF16) {
      r.ks[u] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs.ks, t * 2u, 0, 0));
      r.vs[u] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs.vs, t * 2u, 0, 0));
    } else {
      r.ks[u] = bits_f32(__builtin_amdgcn_raw_buffer_load_b32(rs.ks, t * 4u, 0, 0));
      r.vs[u] = bits_f32(__builtin_amdgcn_raw_buffer_load_b32(rs.vs, t * 4u, 0, 0));
    }
  }
}

// sum over each quad of lanes (one token group), the same bits on its four lanes
__device__ __forceinline__ float attn_quad_sum(float v) {
  v += attn_dpp<0xB1>(v);  // quad_perm [1, 0, 3, 2]
  v += attn_dpp<0x4E>(v);  // quad_perm [2, 3, 0, 1]
  return v;
}

// Workgroups are handed to the XCDs in turn (id mod 8), each XCD with its own L2. Unit u
// and query head g of its group of G map to workgroup (u / 8) * 8 G + 8 g + u mod 8, so the
// G workgroups that read one key/value head's cache share an XCD and are dispatched one
// after another: the later ones find the cache lines in that XCD's L2. The grid holds
// ceil(units / 8) * 8 G workgroups; those past the last unit return at once.
// (Decode over a [16, 8, 2048, 128] cache with 32 query heads: 29.0-29.3 us, against
// 30.4 us with the group's workgroups consecutive in id and so spread over all XCDs.)
constexpr int kAttnXcds = 8;

__host__ __device__ inline void attn_unit_of(int x, int G, int& u, int& g) {
  const int t = x / kAttnXcds;
  g = t % G;
  u = (t / G) * kAttnXcds + x % kAttnXcds;
}

inline uint32_t attn_grid(int64_t units, int64_t G) {
  return (uint32_t)((units + kAttnXcds - 1) / kAttnXcds * kAttnXcds * G);
}

template <int SF16, bool SPLIT>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(4)))
void attention_decode_kernel(AttnArgs a) {
  __shared__ float part[kAttnGroups][kAttnD];
  __shared__ float gmax[kAttnGroups], gsum[kAttnGroups], gw[kAttnGroups], gm;
  // workgroup -> (unit u = (batch, key/value head, split), query head g of the group):
  // attn_unit_of keeps the G query heads of one key/value head on one XCD
  const int G = a.H / a.Hkv;
  int u, g;
  attn_unit_of((int)blockIdx.x, G, u, g);
  if (u >= a.units) return;  // the grid is padded to whole groups of eight units
  const int sp = SPLIT ? u % a.splits : 0;
  const int r = SPLIT ? u / a.splits : u;
  const int b = r / a.Hkv, kvh = r - b * a.Hkv;
  const int h = kvh * G + g;
  const int bh = b * a.H + h;
  const int tid = threadIdx.x, c = tid & 3, tg = tid >> 2;

  // the lane's 32 query dims times the softmax scale, over 16 (exact) for the codes' 16
  float qd[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) qd[i] = (attn_load16(a.q, (int64_t)bh * kAttnD + 32 * c + i, a.q_f16) * a.scale) * 0.0625f;

  const int64_t head = (int64_t)b * a.Hkv + kvh;
  const uint32_t ssz = SF16 ? 2u : 4u;
  const int t_begin = SPLIT ? sp * a.chunk : 0;
  const int n = SPLIT ? max(0, min(a.chunk, a.S - t_begin)) : a.S;
  const int64_t tok0 = head * a.S_cap + t_begin;
  AttnRsrc rs;
  rs.kc = attn_rsrc(a.kc + tok0 * 64, (uint32_t)n * 64u);
  rs.vc = attn_rsrc(a.vc + tok0 * 64, (uint32_t)n * 64u);
  rs.ks = attn_rsrc((const char*)a.ks + tok0 * ssz, (uint32_t)n * ssz);
  rs.vs = attn_rsrc((const char*)a.vs + tok0 * ssz, (uint32_t)n * ssz);

  float m_run = -INFINITY, l_run = 0.0f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.0f;

  // a batch's loads are all issued before any is used, and its first token is in range.
  // Loads are buffer loads range-checked against the workgroup's tokens: a token past them
  // reads zeros and its score is set to -inf (it weighs 0), so no load is predicated.
  for (int t0 = tg; t0 < n; t0 += kAttnU * kAttnGroups) {
    AttnBatch r;
    attn_fetch<SF16>(r, rs, t0, c);
    // keep the batch's loads ahead of its arithmetic (the scheduler would otherwise sink
    // each load to its first use, leaving one token's loads in flight at a time)
    __builtin_amdgcn_sched_barrier(0);
    float sc[kAttnU];
    float bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float kc[8];
        attn_codes16(r.kw[u][j], kc);
#pragma unroll
        for (int i = 0; i < 8; ++i) dot = fmaf(qd[8 * j + i], kc[i], dot);
      }
      dot = attn_quad_sum(dot);
      sc[u] = (t0 + u * kAttnGroups < n) ? dot * r.ks[u] : -INFINITY;
      bmax = fmaxf(bmax, sc[u]);
    }
    const float m_new = fmaxf(m_run, bmax);
    const float corr = __expf(m_run - m_new);
    l_run *= corr;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= corr;
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      const float p = __expf(sc[u] - m_new);
      l_run += p;
      const float pv = (p * r.vs[u]) * 0.0625f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float vc[8];
        attn_codes16(r.vw[u][j], vc);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[8 * j + i] = fmaf(pv, vc[i], acc[8 * j + i]);
      }
    }
    m_run = m_new;
  }

  // ---- merge the 64 groups: weights e^(m_g - M) first, then one output dim per thread
#pragma unroll
  for (int i = 0; i < 32; ++i) part[tg][32 * c + i] = acc[i];
  if (c == 0) {
    gmax[tg] = m_run;
    gsum[tg] = l_run;
  }
  __syncthreads();
  if (tid < kAttnGroups) {
    float mx = gmax[0];
    for (int g = 1; g < kAttnGroups; ++g) mx = fmaxf(mx, gmax[g]);
    gw[tid] = mx == -INFINITY ? 0.0f : __expf(gmax[tid] - mx);
    if (tid == 0) gm = mx;
  }
  __syncthreads();
  if (tid < kAttnD) {
    float o = 0.0f, l = 0.0f;
#pragma unroll 8
    for (int g = 0; g < kAttnGroups; ++g) {
      o = fmaf(part[g][tid], gw[g], o);
      l = fmaf(gsum[g], gw[g], l);
    }
    if constexpr (SPLIT) {
      float* pp = a.part + ((int64_t)bh * a.splits + sp) * (2 + kAttnD);
      pp[2 + tid] = o;
      if (tid == 0) {
        pp[0] = gm;
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
// (split 0 always holds token 0, so M is finite); rounded to the query's format. The
// ranges' maxima and sums are staged in LDS (the threads share the loads), so each
// thread's loop has only independent loads of its output dim.
constexpr int kMergeChunk = 512;  // ranges staged per pass
__global__ __launch_bounds__(kAttnD) void attention_merge_kernel(AttnArgs a) {
  __shared__ float sm[kMergeChunk], sl[kMergeChunk];
  __shared__ float red[kAttnD];
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* pp = a.part + (int64_t)bh * a.splits * (2 + kAttnD);
  float mx = -INFINITY;
  for (int sp = d; sp < a.splits; sp += kAttnD) mx = fmaxf(mx, pp[(int64_t)sp * (2 + kAttnD)]);
  red[d] = mx;
  __syncthreads();
  mx = red[0];
  for (int i = 1; i < kAttnD; ++i) mx = fmaxf(mx, red[i]);
  float o = 0.0f, l = 0.0f;
  for (int base = 0; base < a.splits; base += kMergeChunk) {
    const int cnt = min(kMergeChunk, a.splits - base);
    __syncthreads();  // the previous pass's reads of sm / sl are done
    for (int i = d; i < cnt; i += kAttnD) {
      const float* ps = pp + (int64_t)(base + i) * (2 + kAttnD);
      sm[i] = __expf(ps[0] - mx);  // 0 for a split without tokens (maximum -inf)
      sl[i] = ps[1];
    }
    __syncthreads();
#pragma unroll 8
    for (int i = 0; i < cnt; ++i) {
      const float w = sm[i];
      o = fmaf(pp[(int64_t)(base + i) * (2 + kAttnD) + 2 + d], w, o);
      l = fmaf(sl[i], w, l);
    }
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
  // (the grid is padded by up to 8 heads' worth of workgroups)
  if (batch * heads + 8 * heads > 0x7FFFFFFF || seq_cap > (int64_t{1} << 30) || seq >= (int64_t{1} << 26))
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
  a.units = (int)(batch * a.Hkv * splits);
  const uint32_t grid = attn_grid(a.units, a.H / a.Hkv);
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
  AttnArgs au = a;
  au.units = (int)(batch * kv_heads);
  const dim3 grid(attn_grid(au.units, heads / kv_heads));
  if (a.scale_f16)
    hipLaunchKernelGGL((attention_decode_kernel<1, false>), grid, dim3(kAttnThreads), 0, stream, au);
  else
    hipLaunchKernelGGL((attention_decode_kernel<0, false>), grid, dim3(kAttnThreads), 0, stream, au);
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
  if (batch * heads * splits + 8 * heads > 0x7FFFFFFF) return RBQ_ENOTSUP;
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
  if (batch * heads * splits + 8 * heads > 0x7FFFFFFF) return RBQ_ENOTSUP;
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
