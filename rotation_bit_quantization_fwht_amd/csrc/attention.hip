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

// ---- grouped key/value heads, shared loads: one workgroup per (batch, key/value head,
// set of GW query heads[, range]) takes all GW queries at once, so each cached token is
// loaded once for them (the kernel above loads it once per query head and relies on L2).
// Eight lanes share a token, each taking DL = 16 dims (8 bytes of codes per row); the
// query and output registers take 2 * GW * DL = 64 or 128 per lane. Each token group
// runs the online softmax of the kernel above for each of its GW heads over batches of U
// tokens (256 tokens per batch and workgroup, as above); the code conversion of a token is
// shared by the GW heads. Scores sum over fewer dims per lane and more lanes (16 fused
// multiply-adds and 3 shuffle additions for GW = 4), so their rounding is within the
// kernel above's.
template <int GW>
struct AttnShared {
  static constexpr int L = 8;                       // lanes per token
  static constexpr int DL = kAttnD / L;             // dims per lane
  static constexpr int W = DL / 8;                  // code dwords per lane and token (2)
  static constexpr int NG = kAttnThreads / L;       // token groups
  static constexpr int STRIDE = 256;                // tokens per batch, as in the per-head kernel
  static constexpr int U = STRIDE / NG;             // tokens per group and batch (4 or 8)
};

typedef uint32_t attn_u32x2 __attribute__((ext_vector_type(2)));

// sum over the eight lanes of a token group (quads first, then the two quads of each
// 8-lane half row against each other), the same bits on every lane of the group
__device__ __forceinline__ float attn_octet_sum(float v) {
  v = attn_quad_sum(v);
  return v + attn_dpp<0x141>(v);  // row_half_mirror: lane i <-> 7 - i
}

template <int SF16, bool SPLIT, int GW>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attention_shared_kernel(AttnArgs a) {
  using S = AttnShared<GW>;
  __shared__ float part[S::NG][GW][kAttnD];
  __shared__ float gmax[S::NG][GW], gsum[S::NG][GW], gw[S::NG][GW], gm[GW];
  // workgroup -> (batch, key/value head, set of GW query heads[, range])
  const int sets = (a.H / a.Hkv) / GW;
  const int u = (int)blockIdx.x;
  const int sp = SPLIT ? u % a.splits : 0;
  const int r = SPLIT ? u / a.splits : u;
  const int st = r % sets, bk = r / sets;
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  const int64_t bh0 = (int64_t)b * a.H + (int64_t)kvh * (a.H / a.Hkv) + (int64_t)st * GW;  // first query head
  const int tid = threadIdx.x, c = tid % S::L, tg = tid / S::L;

  // the lane's 16 query dims of each head (two 16-byte loads), times the softmax scale,
  // over 16 (exact) for the codes' 16
  float qd[GW][S::DL];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    const attn_u32x4* qp = (const attn_u32x4*)((const uint16_t*)a.q + (bh0 + g) * kAttnD + S::DL * c);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const attn_u32x4 w = qp[h];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t bits = (w[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
        const float x = a.q_f16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)bits) : bits_f32(bits << 16);
        qd[g][8 * h + i] = (x * a.scale) * 0.0625f;
      }
    }
  }

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

  float m_run[GW], l_run[GW], acc[GW][S::DL];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < S::DL; ++i) acc[g][i] = 0.0f;
  }

  // as in the per-head kernel: range-checked buffer loads (tokens past the range read zeros
  // and score -inf), all of a batch's loads issued before any is used
  for (int t0 = tg; t0 < n; t0 += S::STRIDE) {
    uint32_t kw[S::U][S::W], vw[S::U][S::W];
    float ksc[S::U], vsc[S::U];
#pragma unroll
    for (int v = 0; v < S::U; ++v) {
      const uint32_t t = (uint32_t)(t0 + v * S::NG);
      const attn_u32x2 k2 =
          __builtin_bit_cast(attn_u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs.kc, t * 64u + 8u * c, 0, 0));
      const attn_u32x2 v2 =
          __builtin_bit_cast(attn_u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs.vc, t * 64u + 8u * c, 0, 0));
      kw[v][0] = k2.x; kw[v][1] = k2.y;
      vw[v][0] = v2.x; vw[v][1] = v2.y;
      if constexpr (SF16) {
        ksc[v] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs.ks, t * 2u, 0, 0));
        vsc[v] = (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rs.vs, t * 2u, 0, 0));
      } else {
        ksc[v] = bits_f32(__builtin_amdgcn_raw_buffer_load_b32(rs.ks, t * 4u, 0, 0));
        vsc[v] = bits_f32(__builtin_amdgcn_raw_buffer_load_b32(rs.vs, t * 4u, 0, 0));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the value scale over 16 (exact: a power of two) once per token for the GW heads
#pragma unroll
    for (int v = 0; v < S::U; ++v) vsc[v] *= 0.0625f;
    float sc[GW][S::U];
    float bmax[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) bmax[g] = -INFINITY;
#pragma unroll
    for (int v = 0; v < S::U; ++v) {
      float kc[S::W][8];
#pragma unroll
      for (int j = 0; j < S::W; ++j) attn_codes16(kw[v][j], kc[j]);
      const bool ok = t0 + v * S::NG < n;
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < S::W; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) dot = fmaf(qd[g][8 * j + i], kc[j][i], dot);
        dot = attn_octet_sum(dot);
        sc[g][v] = ok ? dot * ksc[v] : -INFINITY;
        bmax[g] = fmaxf(bmax[g], sc[g][v]);
      }
    }
    float m_new[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      m_new[g] = fmaxf(m_run[g], bmax[g]);
      const float corr = __expf(m_run[g] - m_new[g]);
      l_run[g] *= corr;
#pragma unroll
      for (int i = 0; i < S::DL; ++i) acc[g][i] *= corr;
      m_run[g] = m_new[g];
    }
#pragma unroll
    for (int v = 0; v < S::U; ++v) {
      float vc[S::W][8];
#pragma unroll
      for (int j = 0; j < S::W; ++j) attn_codes16(vw[v][j], vc[j]);
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float p = __expf(sc[g][v] - m_new[g]);
        l_run[g] += p;
        const float pv = p * vsc[v];
#pragma unroll
        for (int j = 0; j < S::W; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[g][8 * j + i] = fmaf(pv, vc[j][i], acc[g][8 * j + i]);
      }
    }
  }

  // ---- merge the token groups of each head, as in the per-head kernel
#pragma unroll
  for (int g = 0; g < GW; ++g)
#pragma unroll
    for (int i = 0; i < S::DL; ++i) part[tg][g][S::DL * c + i] = acc[g][i];
  if (c == 0) {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      gmax[tg][g] = m_run[g];
      gsum[tg][g] = l_run[g];
    }
  }
  __syncthreads();
  if (tid < GW) {
    float mx = gmax[0][tid];
    for (int k = 1; k < S::NG; ++k) mx = fmaxf(mx, gmax[k][tid]);
    gm[tid] = mx;
  }
  __syncthreads();
  for (int e = tid; e < S::NG * GW; e += kAttnThreads) {
    const int k = e / GW, g = e - k * GW;
    gw[k][g] = gm[g] == -INFINITY ? 0.0f : __expf(gmax[k][g] - gm[g]);
  }
  __syncthreads();
  for (int o = tid; o < GW * kAttnD; o += kAttnThreads) {
    const int g = o / kAttnD, d = o - g * kAttnD;
    float acc_o = 0.0f, l = 0.0f;
#pragma unroll 8
    for (int k = 0; k < S::NG; ++k) {
      acc_o = fmaf(part[k][g][d], gw[k][g], acc_o);
      l = fmaf(gsum[k][g], gw[k][g], l);
    }
    const int64_t bh = bh0 + g;
    if constexpr (SPLIT) {
      float* pp = a.part + (bh * a.splits + sp) * (2 + kAttnD);
      pp[2 + d] = acc_o;
      if (d == 0) {
        pp[0] = gm[g];
        pp[1] = l;
      }
    } else {
      acc_o /= l;
      uint16_t bits;
      if (a.q_f16) bits = __builtin_bit_cast(uint16_t, (_Float16)acc_o);
      else bits = (uint16_t)f32_to_bf16(acc_o);
      ((uint16_t*)a.out)[bh * kAttnD + d] = bits;
    }
  }
}

// Query heads per workgroup of the shared-load kernel for G query heads per key/value
// head (0: use the per-head kernel). The shared kernel needs a whole number of sets of
// 2 or 4 heads, and enough workgroups to fill the device: with fewer than 256 it leaves
// CUs idle, where the per-head kernel's G-times larger grid still streams at full rate.
constexpr int64_t kAttnSharedMinWorkgroups = 256;

inline int attn_shared_heads(int64_t G, int64_t units_per_set) {
  const int gw = (G % 4 == 0) ? 4 : ((G % 2 == 0) ? 2 : 0);
  if (gw == 0 || units_per_set * (G / gw) < kAttnSharedMinWorkgroups) return 0;
  return gw;
}

// one launch of the decode kernels over `units` (batch, key/value head[, range]) triples
template <bool SPLIT>
static hipError_t attn_decode_launch(const AttnArgs& a0, int64_t units, hipStream_t stream) {
  AttnArgs a = a0;
  const int64_t G = a.H / a.Hkv;
  const int gw = attn_shared_heads(G, units);
  if (gw) {
    a.units = (int)(units * (G / gw));
    const dim3 grid((uint32_t)a.units);
    if (gw == 4) {
      if (a.scale_f16) hipLaunchKernelGGL((attention_shared_kernel<1, SPLIT, 4>), grid, dim3(kAttnThreads), 0, stream, a);
      else hipLaunchKernelGGL((attention_shared_kernel<0, SPLIT, 4>), grid, dim3(kAttnThreads), 0, stream, a);
    } else {
      if (a.scale_f16) hipLaunchKernelGGL((attention_shared_kernel<1, SPLIT, 2>), grid, dim3(kAttnThreads), 0, stream, a);
      else hipLaunchKernelGGL((attention_shared_kernel<0, SPLIT, 2>), grid, dim3(kAttnThreads), 0, stream, a);
    }
  } else {
    a.units = (int)units;
    const dim3 grid(attn_grid(units, G));
    if (a.scale_f16) hipLaunchKernelGGL((attention_decode_kernel<1, SPLIT>), grid, dim3(kAttnThreads), 0, stream, a);
    else hipLaunchKernelGGL((attention_decode_kernel<0, SPLIT>), grid, dim3(kAttnThreads), 0, stream, a);
  }
  return hipGetLastError();
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
  if (attn_decode_launch<true>(a, batch * a.Hkv * splits, stream) != hipSuccess) return RBQ_EHIP;
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
  return attn_decode_launch<false>(a, batch * kv_heads, stream) == hipSuccess ? RBQ_OK : RBQ_EHIP;
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
