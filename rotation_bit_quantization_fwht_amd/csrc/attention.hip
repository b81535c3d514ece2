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
// One 512-thread workgroup per (batch, head). Sixteen lanes share one cached token: lane c
// takes dims 8c .. 8c + 7, i.e. one dword of codes of the token's 64-byte row, so a wave
// reads four consecutive rows (256 contiguous bytes) per load, and each group loads 16 of
// its tokens before using any of them. The sequence is processed
// in tiles of 2048 tokens with an online softmax: the tile's scores go to LDS, the running
// maximum and sum are updated, and the value rows are accumulated with the tile's
// probabilities. At the end the 32 token groups' partial outputs are summed in LDS.
#include <hip/hip_runtime.h>

#include "../../include/rbq.h"
#include "common.h"
#include "diag.h"
#include "validate.h"

namespace rbq {

struct AttnArgs {
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

constexpr int kAttnThreads = 512;
constexpr int kAttnTile = 2048;   // tokens per tile
constexpr int kAttnD = 128;
constexpr int kAttnU = 16;        // tokens per token group loaded ahead of use

__device__ __forceinline__ float attn_load16(const void* p, int64_t i, int f16) {
  const uint32_t h = ((const uint16_t*)p)[i];
  return f16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)h) : bits_f32(h << 16);
}

__device__ __forceinline__ float attn_scale(const void* p, int64_t i, int f16) {
  return f16 ? attn_load16(p, i, 1) : ((const float*)p)[i];
}

// code i of a dword of packed codes (low nibble first), sign-extended: the builtin's
// result type is unsigned, so it is read as int before the conversion
__device__ __forceinline__ float attn_code(uint32_t w, int i) {
  return (float)(int)__builtin_amdgcn_sbfe(w, 4 * i, 4);
}

// workgroup reduction of one float per thread (max or sum) through LDS
template <bool MAX>
__device__ __forceinline__ float attn_reduce(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = MAX ? fmaxf(v, w) : v + w;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kAttnThreads / 64; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();  // red is reused by the next reduction
  return r;
}

__global__ __launch_bounds__(kAttnThreads) void attention_decode_kernel(AttnArgs a) {
  __shared__ float sc[kAttnTile];
  __shared__ float part[kAttnThreads / 16][kAttnD];
  __shared__ float red[kAttnThreads / 64];
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  const int kvh = h / (a.H / a.Hkv);
  const int tid = threadIdx.x, c = tid & 15, tg = tid >> 4;

  float qd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qd[i] = attn_load16(a.q, (int64_t)bh * kAttnD + 8 * c + i, a.q_f16) * a.scale;

  const int64_t head = (int64_t)b * a.Hkv + kvh;
  const uint32_t* krow = (const uint32_t*)(a.kc + head * a.S_cap * 64);
  const uint32_t* vrow = (const uint32_t*)(a.vc + head * a.S_cap * 64);
  const int64_t srow = head * a.S_cap;

  float m_run = -INFINITY, l_run = 0.0f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;

  for (int s0 = 0; s0 < a.S; s0 += kAttnTile) {
    const int n = min(kAttnTile, a.S - s0);
    // ---- scores of the tile: sixteen lanes per token, eight dims each; kAttnU tokens per
    // token group are loaded before any is used, so their latencies overlap
    float tmax = -INFINITY;
    for (int t0 = tg; t0 < ((n + 15) & ~15); t0 += kAttnU * (kAttnThreads / 16)) {
      uint32_t w[kAttnU];
      float ksv[kAttnU];
#pragma unroll
      for (int u = 0; u < kAttnU; ++u) {
        const int t = t0 + u * (kAttnThreads / 16);
        const bool ok = t < n;
        w[u] = ok ? krow[(int64_t)(s0 + t) * 16 + c] : 0u;
        ksv[u] = ok ? attn_scale(a.ks, srow + s0 + t, a.scale_f16) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kAttnU; ++u) {
        const int t = t0 + u * (kAttnThreads / 16);
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) dot = fmaf(qd[i], attn_code(w[u], i), dot);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
        if (t < n) {
          const float sv = dot * ksv[u];
          if (c == 0) sc[t] = sv;
          tmax = fmaxf(tmax, sv);
        }
      }
    }
    const float m_new = fmaxf(m_run, attn_reduce<true>(tmax, red));  // (its barrier publishes sc)
    // ---- probabilities and the running sum
    float tsum = 0.0f;
    for (int t = tid; t < n; t += kAttnThreads) {
      const float p = __expf(sc[t] - m_new);
      sc[t] = p;
      tsum += p;
    }
    const float corr = __expf(m_run - m_new);  // 0 on the first tile
    l_run = l_run * corr + attn_reduce<false>(tsum, red);
    m_run = m_new;
    // ---- value rows weighted by the probabilities
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= corr;
    for (int t0 = tg; t0 < n; t0 += kAttnU * (kAttnThreads / 16)) {
      uint32_t w[kAttnU];
      float pv[kAttnU];
#pragma unroll
      for (int u = 0; u < kAttnU; ++u) {
        const int t = t0 + u * (kAttnThreads / 16);
        const bool ok = t < n;
        w[u] = ok ? vrow[(int64_t)(s0 + t) * 16 + c] : 0u;
        pv[u] = ok ? sc[t] * attn_scale(a.vs, srow + s0 + t, a.scale_f16) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kAttnU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(pv[u], attn_code(w[u], i), acc[i]);
    }
    __syncthreads();  // the next tile overwrites sc
  }

  // ---- sum the token groups' partial outputs
#pragma unroll
  for (int i = 0; i < 8; ++i) part[tg][8 * c + i] = acc[i];
  __syncthreads();
  if (tid < kAttnD) {
    float o = 0.0f;
#pragma unroll
    for (int g = 0; g < kAttnThreads / 16; ++g) o += part[g][tid];
    o /= l_run;
    uint16_t bits;
    if (a.q_f16) bits = __builtin_bit_cast(uint16_t, (_Float16)o);
    else bits = (uint16_t)f32_to_bf16(o);
    ((uint16_t*)a.out)[(int64_t)bh * kAttnD + tid] = bits;
  }
}

}  // namespace rbq

using namespace rbq;

extern "C" rbq_status attention_decode_int4kv(const void* q, rbq_dtype q_dtype, const uint8_t* k_codes,
                                              const void* k_scales, const uint8_t* v_codes,
                                              const void* v_scales, rbq_dtype scale_dtype, int64_t batch,
                                              int64_t heads, int64_t kv_heads, int64_t seq, int64_t seq_cap,
                                              int64_t head_dim, float softmax_scale, void* out,
                                              hipStream_t stream) {
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
  if (batch * heads > 0x7FFFFFFF || heads > 0x7FFFFFFF || seq_cap > (int64_t{1} << 30)) return RBQ_ENOTSUP;
  AttnArgs a{};
  a.q = q; a.kc = k_codes; a.ks = k_scales; a.vc = v_codes; a.vs = v_scales; a.out = out;
  a.H = (int)heads; a.Hkv = (int)kv_heads; a.S = (int)seq; a.S_cap = (int)seq_cap;
  a.scale = softmax_scale;
  a.q_f16 = q_dtype == RBQ_F16;
  a.scale_f16 = scale_dtype == RBQ_F16;
  if (diag_log())
    fprintf(stderr, "rbq: attention_decode_int4kv B=%lld H=%lld Hkv=%lld S=%lld cap=%lld\n", (long long)batch,
            (long long)heads, (long long)kv_heads, (long long)seq, (long long)seq_cap);
  if (diag_fail_launch()) return RBQ_EHIP;
  hipLaunchKernelGGL(attention_decode_kernel, dim3((uint32_t)(batch * heads)), dim3(kAttnThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}
