// W4A4 GEMM on packed INT4 codes for gfx950:
//   out[m, n] = bf16( sA[m] * sW[n] * sum_k qA[m, k] * qW[n, k] ),  optional int32 sums.
//
// The pages run the rotated, quantized layer as a low-bit GEMM ("SpinQuant: rotate before
// you round", section "Deployment implications"; "SpinQuant Guide: Learned Rotations for
// 4-Bit LLMs", section "The Orthogonal Invariance Principle" and the deployment
// checklist), on INT4 tensor cores of another vendor. gfx950 has no INT4 matrix
// instruction, so the codes are widened to int8 in registers and multiplied with
// v_mfma_i32_32x32x32_i8 (exact int32 accumulation).
//
// Widening: a packed byte holds code k (low nibble) and k+1 (high nibble). For a dword d,
// (d << 4) & 0xF0F0F0F0 gives the even codes and d & 0xF0F0F0F0 the odd codes, each as a
// signed byte equal to 16 * code. Both operands carry the factor 16, so every product is
// 256 times the code product and the sum is 256 times the integer dot product (exact:
// |code| <= 8, so |sum| <= 256 * 64 * K < 2^31 for K <= 65536); it is shifted back by 8. The even/odd split permutes K
// identically in both operands, which leaves the dot product unchanged.
//
// Tiling: a 512-thread workgroup computes a 256 x 256 output tile. Each K step stages
// 128 codes (64 packed bytes) of 256 A rows and 256 W rows in LDS (double buffered,
// 16-byte chunks XOR-swizzled by row so the fragment reads hit distinct banks) while the
// next step's global loads are in flight. The 8 waves form a 2 x 4 grid of 128 (m) x
// 64 (n) wave tiles of 4 x 2 MFMA tiles; W rows are MFMA operand A and A rows operand B,
// so each lane's accumulators hold four consecutive n of one m (8-byte bf16 stores).
#include <hip/hip_runtime.h>

#include "../../include/rbq.h"
#include "common.h"
#include "validate.h"

namespace rbq {

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v16i_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_g __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint8_t* qa;   // [M, K/2]
  const uint8_t* qw;   // [N, K/2]
  const void* sa;      // [M]
  const void* sw;      // [N]
  uint16_t* out;       // bf16 [M, N]
  int32_t* acc;        // optional int32 [M, N]
  int M, N, K;
  int scale_f16;
  int tiles_m, tiles_n;
};

constexpr int kBM = 256, kBN = 256;
constexpr int kStepBytes = 64;            // packed bytes of one row per K step (128 codes)
constexpr int kChunks = kStepBytes / 16;  // 16-byte chunks per row per K step
constexpr int kThreads = 512;

// 16-byte chunk j of row r is stored at chunk j ^ ((r >> 1) & 3): eight consecutive rows
// reading the same chunk then cover all eight 16-byte bank groups
__device__ __forceinline__ int swz(int r, int j) { return r * kChunks + (j ^ ((r >> 1) & 3)); }

__device__ __forceinline__ v4i_t widen(uint32_t d0, uint32_t d1) {
  v4i_t r;
  r[0] = (int)((d0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)(d0 & 0xF0F0F0F0u);
  r[2] = (int)((d1 << 4) & 0xF0F0F0F0u);
  r[3] = (int)(d1 & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ float load_scale(const void* p, int i, int f16) {
  if (f16) return (float)((const _Float16*)p)[i];
  return ((const float*)p)[i];
}

__global__ __launch_bounds__(kThreads) void w4a4_gemm_kernel(GemmArgs g) {
  __shared__ u32x4_g lds[2][2][kBM * kChunks];  // [stage][0: A rows, 1: W rows][chunk]

  // tile order: consecutive workgroups land on different XCDs; give each XCD a contiguous
  // range of tiles, n-major, so the W columns of a range stay in that XCD's L2
  const int ntiles = g.tiles_m * g.tiles_n;
  const int b = blockIdx.x;
  // (a bijection only when the tile count is a multiple of 8; otherwise plain order)
  const int t = (ntiles % 8 == 0) ? (b % 8) * (ntiles / 8) + b / 8 : b;
  const int tn = t / g.tiles_m, tm = t % g.tiles_m;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave & 1) * 128, wn0 = (wave >> 1) * 64;

  const int rowbytes = g.K / 2;
  // global -> LDS: 2 chunks of A rows and 2 of W rows per thread per K step
  const int c0 = tid, c1 = tid + kThreads;
  const int ra0 = c0 / kChunks, ja0 = c0 % kChunks, ra1 = c1 / kChunks, ja1 = c1 % kChunks;
  const int am0 = min(m0 + ra0, g.M - 1), am1 = min(m0 + ra1, g.M - 1);
  const int wn_0 = min(n0 + ra0, g.N - 1), wn_1 = min(n0 + ra1, g.N - 1);
  const uint8_t* pa0 = g.qa + (int64_t)am0 * rowbytes + ja0 * 16;
  const uint8_t* pa1 = g.qa + (int64_t)am1 * rowbytes + ja1 * 16;
  const uint8_t* pw0 = g.qw + (int64_t)wn_0 * rowbytes + ja0 * 16;
  const uint8_t* pw1 = g.qw + (int64_t)wn_1 * rowbytes + ja1 * 16;
  const int sa0 = swz(ra0, ja0), sa1 = swz(ra1, ja1);

  v16i_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16i_t{};

  // fragment rows of this lane: lanes 0..31 and 32..63 read the two halves (g) of a row
  const int fr = lane & 31, fg = lane >> 5;

  const int steps = rowbytes / kStepBytes;
  u32x4_g ga0 = *(const u32x4_g*)pa0, ga1 = *(const u32x4_g*)pa1;
  u32x4_g gw0 = *(const u32x4_g*)pw0, gw1 = *(const u32x4_g*)pw1;
  lds[0][0][sa0] = ga0; lds[0][0][sa1] = ga1;
  lds[0][1][sa0] = gw0; lds[0][1][sa1] = gw1;
  __syncthreads();

  for (int s = 0; s < steps; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < steps;
    if (more) {
      const int off = (s + 1) * kStepBytes;
      ga0 = *(const u32x4_g*)(pa0 + off); ga1 = *(const u32x4_g*)(pa1 + off);
      gw0 = *(const u32x4_g*)(pw0 + off); gw1 = *(const u32x4_g*)(pw1 + off);
    }
    // packed fragments: 32 bytes (two chunks) per row and lane
    u32x4_g fa[4][2], fw[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm0 + i * 32 + fr;
      fa[i][0] = lds[cur][0][swz(r, 2 * fg)];
      fa[i][1] = lds[cur][0][swz(r, 2 * fg + 1)];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wn0 + j * 32 + fr;
      fw[j][0] = lds[cur][1][swz(r, 2 * fg)];
      fw[j][1] = lds[cur][1][swz(r, 2 * fg + 1)];
    }
    // four sub-steps of 32 codes: bytes 8u..8u+7 of the lane's 32 bytes
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v4i_t xa[4], xw[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_g& q = fa[i][u >> 1];
        xa[i] = widen(q[(u & 1) * 2], q[(u & 1) * 2 + 1]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_g& q = fw[j][u >> 1];
        xw[j] = widen(q[(u & 1) * 2], q[(u & 1) * 2 + 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xw[j], xa[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      lds[cur ^ 1][0][sa0] = ga0; lds[cur ^ 1][0][sa1] = ga1;
      lds[cur ^ 1][1][sa0] = gw0; lds[cur ^ 1][1][sa1] = gw1;
    }
    __syncthreads();
  }

  // epilogue: lane holds m = column (lane & 31) of each MFMA tile and, per group q of four
  // accumulators, n = 8 q + 4 (lane >> 5) + {0, 1, 2, 3}
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm0 + i * 32 + fr;
    if (m >= g.M) continue;
    const float sam = load_scale(g.sa, m, g.scale_f16);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn0 + j * 32 + 8 * q + 4 * fg;
        if (n >= g.N) continue;
        int32_t iv[4];
        uint32_t bits[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          iv[e] = acc[i][j][4 * q + e] >> 8;  // exact: every product carried a factor 256
          const float y = ((float)iv[e] * sam) * load_scale(g.sw, n + e, g.scale_f16);
          bits[e] = f32_to_bf16(y);
        }
        *(u32x2*)(g.out + (int64_t)m * g.N + n) = u32x2{bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16)};
        if (g.acc) *(u32x4*)(g.acc + (int64_t)m * g.N + n) = u32x4{(uint32_t)iv[0], (uint32_t)iv[1], (uint32_t)iv[2], (uint32_t)iv[3]};
      }
    }
  }
}

}  // namespace rbq

using namespace rbq;

extern "C" rbq_status w4a4_gemm(const uint8_t* qA, const void* sA, const uint8_t* qW,
                                const void* sW, rbq_dtype scale_dtype, int64_t M, int64_t N,
                                int64_t K, void* out_bf16, int32_t* acc, hipStream_t stream) {
  const rbq_status st = check_gemm(qA, sA, qW, sW, scale_dtype, M, N, K, out_bf16, acc);
  if (st != RBQ_OK || M == 0 || N == 0) return st;
  GemmArgs g{};
  g.qa = qA; g.qw = qW; g.sa = sA; g.sw = sW;
  g.out = (uint16_t*)out_bf16;
  g.acc = acc;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.scale_f16 = scale_dtype == RBQ_F16;
  g.tiles_m = (int)((M + kBM - 1) / kBM);
  g.tiles_n = (int)((N + kBN - 1) / kBN);
  const int64_t ntiles = (int64_t)g.tiles_m * g.tiles_n;
  if (ntiles > 0x7FFFFFFF) return RBQ_ENOTSUP;
  hipLaunchKernelGGL(w4a4_gemm_kernel, dim3((uint32_t)ntiles), dim3(kThreads), 0, stream, g);
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}
