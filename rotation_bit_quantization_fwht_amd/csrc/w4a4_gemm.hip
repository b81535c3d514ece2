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
// |code| <= 8, so |sum| <= 256 * 64 * K < 2^31 for K <= 65536); it is shifted back by 8.
// The even/odd split permutes K identically in both operands, which leaves the dot
// product unchanged.
//
// Tiling: a 512-thread workgroup computes a 256 x 256 output tile. Each K step covers
// 128 codes (64 packed bytes) of 256 A rows and 256 W rows, copied from global memory
// straight into LDS (global_load_lds, 16 bytes per lane, no register staging) through a
// four-stage ring: while step s is multiplied, step s + 1 is already published (its first
// fragments are read before the step ends) and the copies for steps s + 2 and s + 3 are in
// flight; one barrier per step publishes the next step and frees the oldest stage.
// 16-byte chunks are XOR-swizzled by row so the fragment reads hit distinct banks; the
// copy realises the swizzle by choosing which chunk each lane fetches. The 8 waves form a
// 2 x 4 grid of 128 (m) x 64 (n) wave tiles of 4 x 2 MFMA tiles; W rows are MFMA operand
// A and A rows operand B. Within a step the four 32-code sub-steps are software-pipelined:
// the MFMAs of one sub-step overlap the widening of the next one's operands. The epilogue
// stages each wave's bf16 tile through LDS so the output is written in whole 128-byte row
// segments.
#include <hip/hip_runtime.h>

#include "../../include/rbq.h"
#include "common.h"
#include "validate.h"
#include "diag.h"

namespace rbq {

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v16i_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_g __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_g __attribute__((ext_vector_type(2)));

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
  int group;           // group-wise weight scales: codes per group (sw is [N, K / group])
};

constexpr int kBM = 256, kBN = 256;                 // output tile (m x n)
constexpr int kWavesN = kBN / 64;                   // wave grid: 2 (m) x kWavesN (n)
constexpr int kThreads = 128 * kWavesN;
constexpr int kStepBytes = 64;            // packed bytes of one row per K step (128 codes)
constexpr int kChunks = kStepBytes / 16;  // 16-byte chunks per row per K step
constexpr int kStages = 4;
constexpr int kSlotsA = kBM * kChunks;              // 16-byte slots of the A rows of a stage
constexpr int kSlots = (kBM + kBN) * kChunks;       // slots per stage (A rows, then W rows)
constexpr int kLoads = kSlots / kThreads;           // 16-byte copies per thread per step
constexpr int kEpiStride = 144;                     // bytes per staged output row (128 + pad)
static_assert(kSlots % kThreads == 0, "whole copies per thread");
static_assert(2 * kWavesN * 64 * kEpiStride <= kStages * kSlots * 16, "epilogue staging must fit the ring");

// chunk j of row r sits in slot r * 4 + (j ^ key(r)), key(r) = ((r >> 1) ^ (r >> 2)) & 3:
// the 8 (and the 16) consecutive rows that one LDS cycle serves, reading the same chunk,
// then cover 8 (16) distinct 16-byte bank groups
__device__ __forceinline__ int swz_key(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
__device__ __forceinline__ int swz(int r, int j) { return r * kChunks + (j ^ swz_key(r)); }

// Output tile (m, n) of workgroup b for the tiled kernels. Consecutive workgroup ids go
// to different XCDs (b % 8), so XCD x is given the x-th eighth of the tile sequence (a
// bijection when the tile count is a multiple of 8; otherwise plain order). The sequence
// walks groups of 8 tile columns, m-major inside a group: the 32 tiles an XCD runs at once
// then share 4 A row strips and 8 W column strips. For the W4A4 kernel at K = 4096 that is
// 6 MB of operands instead of 9 MB (16 by 2 strips) for its 4 MB L2 (4096 x 11008 x 4096:
// 154.1 -> 152.2 us; 8192 rows: 312.1 -> 301.1 us).
__device__ __forceinline__ int2 tile_of(int b, int tiles_m, int tiles_n) {
  const int ntiles = tiles_m * tiles_n;
  const int t = (ntiles % 8 == 0) ? (b % 8) * (ntiles / 8) + b / 8 : b;
  const int grp = t / (8 * tiles_m), r = t % (8 * tiles_m);
  const int gw = min(8, tiles_n - grp * 8);  // columns in this group
  return int2{r / gw, grp * 8 + r % gw};
}

// One 64-bit shift moves both dwords' even codes up a nibble (d1's low nibble receives d0's
// top one, which the mask clears), one instruction fewer per 16 codes than two 32-bit
// shifts; the compiler splits a 64-bit shift written in C back into two, hence the asm
// (4096 x 11008 x 4096: 151.4 -> 148.4 us, results bit-identical).
__device__ __forceinline__ v4i_t widen(uint32_t d0, uint32_t d1) {
  const uint64_t x0 = ((uint64_t)d1 << 32) | d0;
  uint64_t x;
  asm("v_lshlrev_b64 %0, 4, %1" : "=v"(x) : "v"(x0));
  v4i_t r;
  r[0] = (int)((uint32_t)x & 0xF0F0F0F0u);
  r[1] = (int)(d0 & 0xF0F0F0F0u);
  r[2] = (int)((uint32_t)(x >> 32) & 0xF0F0F0F0u);
  r[3] = (int)(d1 & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ float load_scale(const void* p, int i, int f16) {
  if (f16) return (float)((const _Float16*)p)[i];
  return ((const float*)p)[i];
}

// Wait until at most N of this wave's vector-memory operations are outstanding (they
// retire in issue order), then meet the other waves. The asm is a compiler memory
// barrier as well, so no LDS access moves across it.
template <int N>
__device__ __forceinline__ void wait_copies_and_sync() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// As above, but leaving this wave's L newest LDS reads in flight: for a barrier that frees
// a stage read by older reads only (the loop issues no other LDS or scalar-memory
// operations, so the count covers exactly those reads); the later reads' uses wait for them.
template <int N, int L>
__device__ __forceinline__ void wait_copies_and_sync_keep_reads() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(%1)\n\ts_barrier" ::"n"(N), "n"(L) : "memory");
}

__global__ __launch_bounds__(kThreads) void w4a4_gemm_kernel(GemmArgs g) {
  __shared__ u32x4_g lds[kStages * kSlots];

  // tile order: consecutive workgroups land on different XCDs; give each XCD a contiguous
  // range of tiles
  const int b = blockIdx.x;
  const int2 tt = tile_of(b, g.tiles_m, g.tiles_n);
  const int tm = tt.x, tn = tt.y;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave & 1) * 128, wn0 = (wave >> 1) * 64;

  const int rowbytes = g.K / 2;
  // copy q of a step fills slots q * 512 + tid: lane-contiguous per wave, as the LDS copy
  // requires. Slot -> (row, chunk) inverts the swizzle; rows past the end re-read the last
  // row (their products land in rows/columns that are never stored).
  const uint8_t* src[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int slot = q * kThreads + tid;
    const bool is_a = slot < kSlotsA;
    const int r = (is_a ? slot : slot - kSlotsA) >> 2;
    const int j = (slot & 3) ^ swz_key(r);
    const int row = is_a ? min(m0 + r, g.M - 1) : min(n0 + r, g.N - 1);
    src[q] = (is_a ? g.qa : g.qw) + (int64_t)row * rowbytes + j * 16;
  }
  const int steps = rowbytes / kStepBytes;
  // copies for `step` go to its stage; past the last step they repeat the last step's data
  // into a stage nobody reads again, which keeps the loop free of branches
  auto issue_copies = [&](int step) {
    u32x4_g* dst = lds + (step % kStages) * kSlots + wave * 64;
    const int off = min(step, steps - 1) * kStepBytes;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src[q] + off), (void*)(dst + q * kThreads), 16, 0, 0);
  };

  v16i_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16i_t{};

  // fragment rows of this lane: lanes 0..31 and 32..63 read the two halves (fg) of a row
  const int fr = lane & 31, fg = lane >> 5;
  int fa_slot[4], fw_slot[2];  // slot of chunk 2 fg of each fragment row (chunk c: ^ c)
#pragma unroll
  for (int i = 0; i < 4; ++i) fa_slot[i] = swz(wm0 + i * 32 + fr, 2 * fg);
#pragma unroll
  for (int j = 0; j < 2; ++j) fw_slot[j] = kSlotsA + swz(wn0 + j * 32 + fr, 2 * fg);

  auto read_chunk = [&](int step, int c, u32x4_g (&fa)[4], u32x4_g (&fw)[2]) {
    const u32x4_g* sb = lds + (step % kStages) * kSlots;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = sb[fa_slot[i] ^ c];
#pragma unroll
    for (int j = 0; j < 2; ++j) fw[j] = sb[fw_slot[j] ^ c];
  };

  // four-stage ring. Invariant at the top of iteration s: steps s and s + 1 are published,
  // chunk 0 of step s is in registers and its first sub-step already widened, the copies
  // for step s + 2 may be in flight. Every sub-step's MFMAs overlap the widening of the
  // next sub-step's operands.
  issue_copies(0);
  issue_copies(1);
  issue_copies(2);
  wait_copies_and_sync<kLoads>();  // steps 0 and 1 published
  u32x4_g fa0[4], fw0[2], fa1[4], fw1[2];
  v4i_t xa[2][4], xw[2][2];
  auto widen_sub = [&](const u32x4_g (&fa)[4], const u32x4_g (&fw)[2], int h, v4i_t (&ya)[4], v4i_t (&yw)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ya[i] = widen(fa[i][2 * h], fa[i][2 * h + 1]);
#pragma unroll
    for (int j = 0; j < 2; ++j) yw[j] = widen(fw[j][2 * h], fw[j][2 * h + 1]);
  };
  auto mma_sub = [&](const v4i_t (&ya)[4], const v4i_t (&yw)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(yw[j], ya[i], acc[i][j], 0, 0, 0);
  };
  read_chunk(0, 0, fa0, fw0);
  widen_sub(fa0, fw0, 0, xa[0], xw[0]);
  for (int s = 0; s < steps; ++s) {
    // stage (s + 3) % 4 last held step s - 1, which every wave finished before the
    // barrier that ended the previous iteration
    issue_copies(s + 3);
    read_chunk(s, 1, fa1, fw1);
    // the scheduler would otherwise sink the fragment reads next to their first use and
    // wait for them at once; here they are issued before the MFMAs they overlap
    __builtin_amdgcn_sched_barrier(0);
    mma_sub(xa[0], xw[0]);
    widen_sub(fa0, fw0, 1, xa[1], xw[1]);
    mma_sub(xa[1], xw[1]);
    widen_sub(fa1, fw1, 0, xa[0], xw[0]);
    read_chunk(s + 1, 0, fa0, fw0);  // (after the last step: a stale stage, never used)
    __builtin_amdgcn_sched_barrier(0);
    mma_sub(xa[0], xw[0]);
    widen_sub(fa1, fw1, 1, xa[1], xw[1]);
    mma_sub(xa[1], xw[1]);
    widen_sub(fa0, fw0, 0, xa[0], xw[0]);
    // publish step s + 2: this wave's copies for it are done when at most those of step
    // s + 3 are in flight. The barrier also frees step s's stage for the copies of step
    // s + 4: its reads (chunk 1 above, chunk 0 in the previous iteration) must be done,
    // while the 6 reads of step s + 1's chunk 0 just issued may stay in flight.
    wait_copies_and_sync_keep_reads<kLoads, 6>();
  }

  // epilogue. Lane holds m = column (lane & 31) of each MFMA tile and, per group q of four
  // accumulators, n = 8 q + 4 (lane >> 5) + {0, 1, 2, 3}.
  if (g.acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm0 + i * 32 + fr;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn0 + j * 32 + 8 * q + 4 * fg;
          if (n >= g.N) continue;
          // exact: every product carried a factor 256
          *(u32x4*)(g.acc + (int64_t)m * g.N + n) =
              u32x4{(uint32_t)(acc[i][j][4 * q] >> 8), (uint32_t)(acc[i][j][4 * q + 1] >> 8),
                    (uint32_t)(acc[i][j][4 * q + 2] >> 8), (uint32_t)(acc[i][j][4 * q + 3] >> 8)};
        }
    }
  }
  float swv[2][4][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        swv[j][q][e] = load_scale(g.sw, min(n0 + wn0 + j * 32 + 8 * q + 4 * fg + e, g.N - 1), g.scale_f16);

  // bf16 results go through this wave's private LDS rows (64 m x 64 n per half), then out
  // as 16-byte pieces, eight lanes per 128-byte row segment
  wait_copies_and_sync<0>();  // every wave is done with the ring
  char* stage = (char*)lds + wave * 64 * kEpiStride;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * hh + ii;
      const float sam = load_scale(g.sa, min(m0 + wm0 + i * 32 + fr, g.M - 1), g.scale_f16);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = ((float)(acc[i][j][4 * q + e] >> 8) * sam) * swv[j][q][e];
          *(u32x2*)(stage + (ii * 32 + fr) * kEpiStride + (j * 32 + 8 * q + 4 * fg) * 2) =
              u32x2{f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3])};
        }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rloc = it * 8 + (lane >> 3);
      const u32x4 v = *(const u32x4*)(stage + rloc * kEpiStride + (lane & 7) * 16);
      const int m = m0 + wm0 + hh * 64 + rloc;
      const int n = n0 + wn0 + (lane & 7) * 8;
      // nontemporal: the whole output of a wave of tiles goes out at once, and it is not
      // read again; streamed, it evicts less of the operand rows the next tiles read
      if (m < g.M && n < g.N)
        __builtin_nontemporal_store(u32x4_g{v.x, v.y, v.z, v.w}, (u32x4_g*)(g.out + (int64_t)m * g.N + n));
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// ------------------------------------------------------------------------------ W4A8
// INT8 activation codes (one byte per code, scale max/127 per token) times packed INT4
// weight codes. Same tiling as above; per K step (128 codes) an A row brings 128 bytes
// (8 chunks) and a W row 64 bytes. Each 32-code sub-step takes one 16-byte A chunk per
// lane; its bytes are permuted into the order the W widening produces (even codes of the
// first 8, odd codes of the first 8, even of the next 8, odd of the next 8), so both MFMA
// operands list the same k in the same positions. W carries the factor 16, so the sums
// are 16 times the integer dot product (|sum| <= 16 * 128 * 8 * K < 2^31 for K <= 65536)
// and are shifted back by 4.
constexpr int kA8Chunks = 8;                                  // A chunks per row per step
constexpr int kA8SlotsA = kBM * kA8Chunks;                    // 2048
constexpr int kA8Slots = kA8SlotsA + kBN * kChunks;           // 3072 per stage (48 KB)
constexpr int kA8Loads = kA8Slots / kThreads;                 // 6 copies per thread
constexpr int kA8Stages = 3;
constexpr int kA8Lds = (kA8Stages * kA8Slots * 16 > 8 * 64 * kEpiStride) ? kA8Stages * kA8Slots * 16 : 8 * 64 * kEpiStride;
static_assert(kA8Slots % kThreads == 0, "whole copies per thread");
static_assert(kA8Loads == 6, "the wait counts below assume six copies per thread and step");

// chunk j of A row r: slot r * 8 + (j ^ key8(r)), key8(r) = ((r >> 1) ^ (r << 2)) & 7, so
// 8 and 16 consecutive rows reading one chunk fall in distinct 16-byte bank groups
__device__ __forceinline__ int swz_key8(int r) { return ((r >> 1) ^ (r << 2)) & 7; }
__device__ __forceinline__ int swz8(int r, int j) { return r * kA8Chunks + (j ^ swz_key8(r)); }

// bytes c0..c15 of one A chunk -> [c0 c2 c4 c6 | c1 c3 c5 c7 | c8 c10 c12 c14 | c9 c11 c13 c15]
__device__ __forceinline__ v4i_t order_like_widen(const u32x4_g& q) {
  v4i_t r;
  r[0] = (int)__builtin_amdgcn_perm(q[1], q[0], 0x06040200u);
  r[1] = (int)__builtin_amdgcn_perm(q[1], q[0], 0x07050301u);
  r[2] = (int)__builtin_amdgcn_perm(q[3], q[2], 0x06040200u);
  r[3] = (int)__builtin_amdgcn_perm(q[3], q[2], 0x07050301u);
  return r;
}

__global__ __launch_bounds__(kThreads) void w4a8_gemm_kernel(GemmArgs g) {
  __shared__ u32x4_g lds[kA8Lds / 16];
  const int b = blockIdx.x;
  const int2 tt = tile_of(b, g.tiles_m, g.tiles_n);  // as in w4a4_gemm_kernel
  const int tm = tt.x, tn = tt.y;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave & 1) * 128, wn0 = (wave >> 1) * 64;
  const int abytes = g.K, wbytes = g.K / 2;       // row bytes of A (int8) and W (packed)
  const int steps = g.K / 128;

  const uint8_t* src[kA8Loads];
  int src_step[kA8Loads];                           // bytes per step of that source row
#pragma unroll
  for (int q = 0; q < kA8Loads; ++q) {
    const int slot = q * kThreads + tid;
    if (slot < kA8SlotsA) {
      const int r = slot >> 3;
      const int j = (slot & 7) ^ swz_key8(r);
      src[q] = g.qa + (int64_t)min(m0 + r, g.M - 1) * abytes + j * 16;
      src_step[q] = 128;
    } else {
      const int r = (slot - kA8SlotsA) >> 2;
      const int j = (slot & 3) ^ swz_key(r);
      src[q] = g.qw + (int64_t)min(n0 + r, g.N - 1) * wbytes + j * 16;
      src_step[q] = 64;
    }
  }
  auto issue_copies = [&](int step) {
    u32x4_g* dst = lds + (step % kA8Stages) * kA8Slots + wave * 64;
    const int st = min(step, steps - 1);
#pragma unroll
    for (int q = 0; q < kA8Loads; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src[q] + st * src_step[q]), (void*)(dst + q * kThreads), 16, 0, 0);
  };

  v16i_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16i_t{};

  // lane (fr, fg) covers codes 64 fg .. 64 fg + 63 of each step: W chunks 2 fg, 2 fg + 1
  // (two sub-steps each), A chunks 4 fg .. 4 fg + 3 (one per sub-step)
  const int fr = lane & 31, fg = lane >> 5;
  int fa_row[4], fw_slot[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa_row[i] = wm0 + i * 32 + fr;
#pragma unroll
  for (int j = 0; j < 2; ++j) fw_slot[j] = kA8SlotsA + swz(wn0 + j * 32 + fr, 2 * fg);
  auto read_a = [&](int step, int u, u32x4_g (&fa)[4]) {
    const u32x4_g* sb = lds + (step % kA8Stages) * kA8Slots;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = sb[swz8(fa_row[i], 4 * fg + u)];
  };
  auto read_w = [&](int step, int c, u32x4_g (&fw)[2]) {
    const u32x4_g* sb = lds + (step % kA8Stages) * kA8Slots;
#pragma unroll
    for (int j = 0; j < 2; ++j) fw[j] = sb[fw_slot[j] ^ c];
  };
  auto prep = [&](const u32x4_g (&fa)[4], const u32x4_g (&fw)[2], int h, v4i_t (&ya)[4], v4i_t (&yw)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ya[i] = order_like_widen(fa[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) yw[j] = widen(fw[j][2 * h], fw[j][2 * h + 1]);
  };
  auto mma_sub = [&](const v4i_t (&ya)[4], const v4i_t (&yw)[2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(yw[j], ya[i], acc[i][j], 0, 0, 0);
  };

  // three-stage ring; at the top of iteration s steps s and s + 1 are published and the
  // operands of sub-step 0 of step s are ready
  issue_copies(0);
  issue_copies(1);
  wait_copies_and_sync<0>();
  u32x4_g fa[4], fw0[2], fw1[2];
  v4i_t xa[2][4], xw[2][2];
  read_a(0, 0, fa);
  read_w(0, 0, fw0);
  prep(fa, fw0, 0, xa[0], xw[0]);
  for (int s = 0; s < steps; ++s) {
    issue_copies(s + 2);  // its stage last held step s - 1, finished before the last barrier
    // (each sched_barrier keeps the fragment reads ahead of the MFMAs they overlap)
    read_a(s, 1, fa);
    read_w(s, 1, fw1);
    __builtin_amdgcn_sched_barrier(0);
    mma_sub(xa[0], xw[0]);
    prep(fa, fw0, 1, xa[1], xw[1]);
    read_a(s, 2, fa);
    __builtin_amdgcn_sched_barrier(0);
    mma_sub(xa[1], xw[1]);
    prep(fa, fw1, 0, xa[0], xw[0]);
    read_a(s, 3, fa);
    __builtin_amdgcn_sched_barrier(0);
    mma_sub(xa[0], xw[0]);
    prep(fa, fw1, 1, xa[1], xw[1]);
    read_a(s + 1, 0, fa);   // (after the last step: a stale stage, never used)
    read_w(s + 1, 0, fw0);
    __builtin_amdgcn_sched_barrier(0);
    mma_sub(xa[1], xw[1]);
    prep(fa, fw0, 0, xa[0], xw[0]);
    wait_copies_and_sync<0>();  // publishes step s + 2
  }

  if (g.acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm0 + i * 32 + fr;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn0 + j * 32 + 8 * q + 4 * fg;
          if (n >= g.N) continue;
          *(u32x4*)(g.acc + (int64_t)m * g.N + n) =
              u32x4{(uint32_t)(acc[i][j][4 * q] >> 4), (uint32_t)(acc[i][j][4 * q + 1] >> 4),
                    (uint32_t)(acc[i][j][4 * q + 2] >> 4), (uint32_t)(acc[i][j][4 * q + 3] >> 4)};
        }
    }
  }
  float swv[2][4][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        swv[j][q][e] = load_scale(g.sw, min(n0 + wn0 + j * 32 + 8 * q + 4 * fg + e, g.N - 1), g.scale_f16);
  wait_copies_and_sync<0>();
  char* stage = (char*)lds + wave * 64 * kEpiStride;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * hh + ii;
      const float sam = load_scale(g.sa, min(m0 + wm0 + i * 32 + fr, g.M - 1), g.scale_f16);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = ((float)(acc[i][j][4 * q + e] >> 4) * sam) * swv[j][q][e];
          *(u32x2*)(stage + (ii * 32 + fr) * kEpiStride + (j * 32 + 8 * q + 4 * fg) * 2) =
              u32x2{f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3])};
        }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int rloc = it * 8 + (lane >> 3);
      const u32x4 v = *(const u32x4*)(stage + rloc * kEpiStride + (lane & 7) * 16);
      const int m = m0 + wm0 + hh * 64 + rloc;
      const int n = n0 + wn0 + (lane & 7) * 8;
      // nontemporal: the whole output of a wave of tiles goes out at once, and it is not
      // read again; streamed, it evicts less of the operand rows the next tiles read
      if (m < g.M && n < g.N)
        __builtin_nontemporal_store(u32x4_g{v.x, v.y, v.z, v.w}, (u32x4_g*)(g.out + (int64_t)m * g.N + n));
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}


// ------------------------------------------------------------- W4A8, group-wise W scales
// out[m, n] = bf16( sA[m] * sum_g sW[n, g] * sum_{k in group g} qA[m, k] * qW[n, k] ):
// the int32 sums of each group of G codes (G a power of two dividing K, G >= 32) are
// exact, and are scaled and added in fp32 when the group ends. A 512-thread workgroup
// computes a 128 (m) x 256 (n) tile; its eight waves form a 2 x 4 grid of 64 x 64 wave
// tiles of 2 x 2 MFMA tiles, with int32 accumulators for the current group and fp32 ones
// for the finished groups. Each 32-code sub-step covers 32 consecutive codes (32u .. 32u +
// 31 of a 128-code step), so every group boundary falls between sub-steps (FS sub-steps
// per group: 1 for groups of 32, 2 for 64, and whole steps for 128 or more): lane half fg
// takes codes 16 fg .. 16 fg + 15 of it, one 16-byte A chunk and one 8-byte half of the W
// chunk. Copies go through a four-stage LDS ring as in the W4A4 kernel (A chunks swizzled
// by key8, W by key; the copies of a step are issued two steps ahead), and the operand
// reads of the next sub-step (and of the next step's first one) overlap the MFMAs of the
// current one. With groups of 64 codes or more, two sub-steps are read as one: lane half fg
// takes the whole 16-byte W chunk 2 v + fg of half-step v (codes 64 v + 32 fg .. + 31) and
// the two A chunks of the same codes, and runs one MFMA per 16 of them. Each MFMA's codes
// then lie in one 64-code block, so in one group; the W reads are half as many and, whole
// chunks under the row key, free of bank conflicts (an 8-byte read of half a chunk puts the
// 32 lanes of a pass on half the banks).
//
// A rows are MFMA operand A and W rows operand B, so each lane holds one output column n
// per W block (and sixteen rows m): the fold at a group's end multiplies the lane's
// accumulators by one of two group scales, which the lane loads itself a step ahead. acc
// holds 16 x the group sum (W is widened to 16 x code), so the fp32 accumulator collects
// 16 x sum_g sW * sum_g; the epilogue multiplies by 1/16 (exact) and sA. The next group's
// first MFMAs take a zero accumulator instead of clearing acc.
constexpr int kGBM = 128, kGBN = 256, kGThreads = 512;
constexpr int kGSlotsA = kGBM * kA8Chunks;                // 1024
constexpr int kGSlots = kGSlotsA + kGBN * kChunks;        // 2048 per stage (32 KB)
constexpr int kGLoads = kGSlots / kGThreads;              // 4 copies per thread
constexpr int kGStages = 4;
constexpr int kGRing = kGStages * kGSlots * 16;           // 128 KB
static_assert(kGSlots % kGThreads == 0, "whole copies per thread");
static_assert(8 * 64 * kEpiStride <= kGRing, "the epilogue staging must fit the ring");

typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit data, no swizzle, range-checked

// FS: sub-steps per group (1, 2), or 4 for groups of 128 codes or more
template <int SF16, int FS>
__global__ __launch_bounds__(kGThreads) void w4a8_gemm_grouped_kernel(GemmArgs g) {
  __shared__ u32x4_g lds[kGRing / 16];
  const int b = blockIdx.x;
  const int2 tt = tile_of(b, g.tiles_m, g.tiles_n);  // as in w4a4_gemm_kernel
  const int tm = tt.x, tn = tt.y;
  const int m0 = tm * kGBM, n0 = tn * kGBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave & 1) * 64, wn0 = (wave >> 1) * 64;
  const int abytes = g.K, wbytes = g.K / 2;
  const int steps = g.K / 128;
  const int ngroups = g.K / g.group;
  // groups of 128 codes or more: steps per group (a power of two), as a mask and a shift
  const int spg_mask = FS == 4 ? g.group / 128 - 1 : 0;
  const int spg_log = FS == 4 ? __builtin_ctz(g.group / 128) : 0;

  // copies q = 0, 1 fill A slots and q = 2, 3 W slots, as buffer loads into LDS: each
  // lane keeps a 32-bit offset from the tile's first row (rows clamped to the matrix) and
  // the step offset is a uniform register, so the copies hold no address registers
  static_assert(kGSlotsA == 2 * kGThreads, "copies 0 and 1 are the A rows");
  uint32_t coff[kGLoads];
#pragma unroll
  for (int q = 0; q < kGLoads; ++q) {
    const int slot = q * kGThreads + tid;
    if (q < 2) {
      const int r = slot >> 3;
      const int j = (slot & 7) ^ swz_key8(r);
      coff[q] = (uint32_t)((min(m0 + r, g.M - 1) - m0) * abytes + j * 16);
    } else {
      const int r = (slot - kGSlotsA) >> 2;
      const int j = (slot & 3) ^ swz_key(r);
      coff[q] = (uint32_t)((min(n0 + r, g.N - 1) - n0) * wbytes + j * 16);
    }
  }
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.qa + (int64_t)m0 * abytes), (short)0, min(kGBM, g.M - m0) * abytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(g.qw + (int64_t)n0 * wbytes), (short)0, min(kGBN, g.N - n0) * wbytes, kBufferWord3);
  auto issue_copies = [&](int step) {
    u32x4_g* dst = lds + (step % kGStages) * kGSlots + wave * 64;
    const int st = min(step, steps - 1);
#pragma unroll
    for (int q = 0; q < kGLoads; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 2 ? arsrc : wrsrc, (lds_ptr_t)(dst + q * kGThreads), 16,
                                               coff[q], q < 2 ? st * 128 : st * 64, 0, 0);
  };

  v16i_t acc[2][2];
  float facc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = v16i_t{};
#pragma unroll
      for (int e = 0; e < 16; ++e) facc[i][j][e] = 0.0f;
    }

  const int fr = lane & 31, fg = lane >> 5;
  int fa_row[2], fw_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) fa_row[i] = wm0 + i * 32 + fr;
#pragma unroll
  for (int j = 0; j < 2; ++j) fw_row[j] = wn0 + j * 32 + fr;

  // the lane's two output columns n = n0 + wn0 + 32 j + fr: their group scales, loaded as
  // bits (a buffer load: a persistent lane offset and a uniform group offset, so no address
  // registers that later instructions would have to wait for) and converted at the fold
  constexpr int ssz = SF16 ? 2 : 4;
  const int nw = min(n0 + wn0, g.N - 1);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)g.sw + (int64_t)nw * ngroups * ssz), (short)0, 64 * ngroups * ssz, kBufferWord3);
  uint32_t soff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) soff[j] = (uint32_t)((min(n0 + wn0 + 32 * j + fr, g.N - 1) - nw) * ngroups * ssz);
  auto load_sw = [&](int j, int grp) -> uint32_t {
    const int go = min(grp, ngroups - 1) * ssz;
    if constexpr (SF16) return __builtin_amdgcn_raw_buffer_load_b16(srsrc, soff[j], go, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(srsrc, soff[j], go, 0);
  };
  auto sw_value = [&](uint32_t bits) {
    return SF16 ? (float)__builtin_bit_cast(_Float16, (uint16_t)bits) : bits_f32(bits);
  };

  // acc[i][j] element 4q + e is output (m = wm0 + 32 i + 8 q + 4 fg + e, n = wn0 + 32 j + fr)
  auto fold = [&](const uint32_t (&bits)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float sw = sw_value(bits[j]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) facc[i][j][e] = fmaf((float)acc[i][j][e], sw, facc[i][j][e]);
    }
  };

  // lane half fg reads the 8 bytes (16 codes) of the W chunk it uses. The second read's
  // address is made opaque so the two are not merged into one ds_read2, which the
  // compiler would make wait for the copies in flight.
  auto read_sub = [&](int step, int u, u32x4_g (&ca)[2], u32x2_g (&cw)[2]) {
    const u32x4_g* sb = lds + (step % kGStages) * kGSlots;
#pragma unroll
    for (int i = 0; i < 2; ++i) ca[i] = sb[swz8(fa_row[i], 2 * u + fg)];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t slot = (uint32_t)(kGSlotsA + swz(fw_row[j], u));
      if (j) asm volatile("" : "+v"(slot));
      cw[j] = ((const u32x2_g*)(sb + slot))[fg];
    }
  };
  auto prep = [&](const u32x4_g (&ca)[2], const u32x2_g (&cw)[2], v4i_t (&ya)[2], v4i_t (&yw)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) ya[i] = order_like_widen(ca[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) yw[j] = widen(cw[j][0], cw[j][1]);
  };
  auto mma_sub = [&](const v4i_t (&ya)[2], const v4i_t (&yw)[2], bool fresh) {
    if (fresh) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ya[i], yw[j], v16i_t{}, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ya[i], yw[j], acc[i][j], 0, 0, 0);
    }
  };

  // half-step v (groups of 64 codes or more): whole chunks, one MFMA per 16 codes of a lane
  auto read_half = [&](int step, int v, u32x4_g (&da)[2][2], u32x4_g (&dw)[2]) {
    const u32x4_g* sb = lds + (step % kGStages) * kGSlots;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) da[i][h] = sb[swz8(fa_row[i], 4 * v + 2 * fg + h)];
#pragma unroll
    for (int j = 0; j < 2; ++j) dw[j] = sb[kGSlotsA + swz(fw_row[j], 2 * v + fg)];
  };
  auto prep_half = [&](const u32x4_g (&da)[2][2], const u32x4_g (&dw)[2], v4i_t (&ya)[2][2], v4i_t (&yw)[2][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 2; ++i) ya[h][i] = order_like_widen(da[i][h]);
#pragma unroll
      for (int j = 0; j < 2; ++j) yw[h][j] = widen(dw[j][2 * h], dw[j][2 * h + 1]);
    }
  };

  // scales of the groups the current step ends (FS < 4: 4 / FS groups; FS = 4: the one
  // group that ends with some step), loaded a step ahead
  constexpr int GPS = FS == 4 ? 1 : 4 / FS;
  uint32_t swc[GPS][2];
#pragma unroll
  for (int gi = 0; gi < GPS; ++gi)
#pragma unroll
    for (int j = 0; j < 2; ++j) swc[gi][j] = load_sw(j, gi);

  // four-stage ring: at the top of iteration s steps s and s + 1 are published, the
  // operands of sub-step 0 of step s are read and the copies for step s + 2 may be in
  // flight
  issue_copies(0);
  issue_copies(1);
  issue_copies(2);
  wait_copies_and_sync<kGLoads>();  // steps 0 and 1 published
  u32x4_g ca[2];
  u32x2_g cw[2];
  v4i_t ya[2], yw[2];
  u32x4_g da[2][2], dw[2];
  if constexpr (FS == 1) read_sub(0, 0, ca, cw);
  else read_half(0, 0, da, dw);
  for (int s = 0; s < steps; ++s) {
    // the scales the next step needs, loaded a whole step before the barrier waits for them
    const bool fresh = FS == 4 ? (s & spg_mask) == 0 : true;       // a group starts with this step
    const bool ends = FS == 4 ? ((s + 1) & spg_mask) == 0 : true;  // and one ends with it
    uint32_t swn[GPS][2];
#pragma unroll
    for (int gi = 0; gi < GPS; ++gi)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        swn[gi][j] = !ends ? 0u : load_sw(j, FS == 4 ? ((s + 1) >> spg_log) : (s + 1) * GPS + gi);
    issue_copies(s + 3);  // its stage last held step s - 1, finished before the last barrier
    if constexpr (FS == 1) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        prep(ca, cw, ya, yw);
        if (u < 3) read_sub(s, u + 1, ca, cw);
        else read_sub(s + 1, 0, ca, cw);  // (after the last step: a stale stage, never used)
        mma_sub(ya, yw, true);
        // (kept in place: spread among later MFMAs, the fold's temporaries would hold
        // more registers than the workgroup has)
        __builtin_amdgcn_sched_barrier(0);
        fold(swc[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        v4i_t yah[2][2], ywh[2][2];
        prep_half(da, dw, yah, ywh);
        if (v == 0) read_half(s, 1, da, dw);
        else read_half(s + 1, 0, da, dw);  // (after the last step: a stale stage, never used)
        mma_sub(yah[0], ywh[0], FS == 4 ? (fresh && v == 0) : true);
        mma_sub(yah[1], ywh[1], false);
        if constexpr (FS == 2) {  // a group per half-step
          __builtin_amdgcn_sched_barrier(0);
          fold(swc[v]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (ends) {
      if constexpr (FS == 4) fold(swc[0]);
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi)
#pragma unroll
        for (int j = 0; j < 2; ++j) swc[gi][j] = swn[gi][j];
    }
    // publish step s + 2: this wave's copies for it (and everything issued before them)
    // are done when at most those of step s + 3 are in flight
    wait_copies_and_sync<kGLoads>();
  }
  wait_copies_and_sync<0>();  // no copy is in flight when the ring becomes the staging area

  // epilogue: scale, round, stage each wave's 64 x 64 bf16 tile in LDS (the ring is free
  // after the barrier above; a lane writes its column of each 32-row block, 16 bits at a
  // time) and write whole 128-byte row segments
  char* stage = (char*)lds + wave * 64 * kEpiStride;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ml = i * 32 + 8 * q + 4 * fg + e;
        const float sam = load_scale(g.sa, min(m0 + wm0 + ml, g.M - 1), g.scale_f16);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          *(uint16_t*)(stage + ml * kEpiStride + (j * 32 + fr) * 2) =
              (uint16_t)f32_to_bf16((facc[i][j][4 * q + e] * 0.0625f) * sam);
      }
  __builtin_amdgcn_wave_barrier();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int rloc = it * 8 + (lane >> 3);
    const u32x4 v = *(const u32x4*)(stage + rloc * kEpiStride + (lane & 7) * 16);
    const int m = m0 + wm0 + rloc;
    const int n = n0 + wn0 + (lane & 7) * 8;
    if (m < g.M && n < g.N) *(u32x4*)(g.out + (int64_t)m * g.N + n) = v;
  }
}

// ------------------------------------------------------------------ few tokens (decode)
// With at most 64 tokens (M) the 256 x 256 tiles leave almost every CU idle (43 workgroups
// for N = 11008, each doing 256 rows of work for the few real ones), while the work is
// bound by streaming the weights once. Here a workgroup of four waves takes 16 weight rows
// (n) and all M tokens in blocks of 16, and the waves split K: wave w takes the 128-code
// steps w, w + 4, w + 8, ... In a step, lane (r, g) = (lane & 15, lane >> 4) loads 16
// bytes of weight row n0 + r (codes 128 s + 32 g .. + 31: a row's four lanes read 64
// contiguous bytes) and the same codes of token r of each block, and runs two
// v_mfma_i32_16x16x64_i8 (16 codes per lane each) per block, with the operands widened as
// in the tiled kernel (the same products, the same int32 sums). All weight and activation
// loads of a chunk of steps are issued before its MFMAs. The waves' sums are added in LDS
// (exact) and wave 0 scales and stores them with the tiled kernel's epilogue arithmetic.
constexpr int kSmallMaxM = 64;
constexpr int kSmallWaves = 4;

template <bool A8, int TB>
__global__ __launch_bounds__(64 * kSmallWaves) void gemm_small_m_kernel(GemmArgs g) {
  constexpr int AV = A8 ? 2 : 1;                             // 16-byte activation loads per step
  // steps per chunk: 8 (a wave's share of K = 4096) for one token block, fewer for more
  // blocks (their activation registers)
  constexpr int C = 8 / TB;
  __shared__ int32_t red[kSmallWaves - 1][TB][4][64];         // waves 1 .. 3's sums, [value][lane]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = (int)blockIdx.x * 16;
  const int r = lane & 15, kg = lane >> 4;
  // rows past the end re-read the last row (their sums are never stored)
  const uint8_t* wp = g.qw + (int64_t)min(n0 + r, g.N - 1) * (g.K / 2) + 16 * kg;
  const int64_t abytes = A8 ? g.K : g.K / 2;
  const uint8_t* ap[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) ap[t] = g.qa + (int64_t)min(t * 16 + r, g.M - 1) * abytes + 16 * AV * kg;

  v4i_t acc[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) acc[t] = v4i_t{};
  const int steps = g.K / 128;
  for (int s0 = wave; s0 < steps; s0 += kSmallWaves * C) {
    u32x4_g w[C], a[TB][C][AV];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      // steps past the end load the last step again (never used)
      const int s = min(s0 + kSmallWaves * c, steps - 1);
      w[c] = *(const u32x4_g*)(wp + (int64_t)s * 64);
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int v = 0; v < AV; ++v) a[t][c][v] = *(const u32x4_g*)(ap[t] + (int64_t)s * 64 * AV + 16 * v);
    }
    // every load of the chunk is issued before the first MFMA (the scheduler would
    // otherwise interleave them and wait sooner)
    __builtin_amdgcn_sched_barrier(0);
    // straight-line from the loads to the MFMAs (a branch per step would let the compiler
    // sink each step's loads next to their use, one memory latency per step): steps past
    // the end take part with their weight codes masked to zero
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint32_t keep = (s0 + kSmallWaves * c < steps) ? 0xFFFFFFFFu : 0u;
      const v4i_t yw0 = widen(w[c][0] & keep, w[c][1] & keep), yw1 = widen(w[c][2] & keep, w[c][3] & keep);
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        v4i_t ya0, ya1;
        if constexpr (A8) {
          ya0 = order_like_widen(a[t][c][0]);
          ya1 = order_like_widen(a[t][c][1]);
        } else {
          ya0 = widen(a[t][c][0][0], a[t][c][0][1]);
          ya1 = widen(a[t][c][0][2], a[t][c][0][3]);
        }
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(yw0, ya0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(yw1, ya1, acc[t], 0, 0, 0);
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int k = 0; k < 4; ++k) red[wave - 1][t][k][lane] = acc[t][k];
  }
  __syncthreads();
  if (wave != 0) return;
  // lane holds token m = 16 t + r and weight rows n = n0 + 4 kg + e, e = 0 .. 3
  constexpr int SH = A8 ? 4 : 8;  // the codes' factor 16 (W only) or 256 (both operands)
  const int n = n0 + 4 * kg;
  if (n >= g.N) return;  // N is a multiple of 8, so n .. n + 3 are all in range
  float swv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) swv[e] = load_scale(g.sw, n + e, g.scale_f16);
#pragma unroll
  for (int t = 0; t < TB; ++t) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int v = 0; v < kSmallWaves - 1; ++v) acc[t][k] += red[v][t][k][lane];
    const int m = t * 16 + r;
    if (m >= g.M) continue;
    if (g.acc)
      *(u32x4*)(g.acc + (int64_t)m * g.N + n) =
          u32x4{(uint32_t)(acc[t][0] >> SH), (uint32_t)(acc[t][1] >> SH), (uint32_t)(acc[t][2] >> SH),
                (uint32_t)(acc[t][3] >> SH)};
    const float sam = load_scale(g.sa, m, g.scale_f16);
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = ((float)(acc[t][e] >> SH) * sam) * swv[e];
    *(u32x2*)(g.out + (int64_t)m * g.N + n) = u32x2{f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3])};
  }
}

// Few tokens with group-wise weight scales (w4a8_gemm_grouped, M <= 64): a workgroup of
// four waves takes 32 weight rows and the tokens in blocks of 32. Tokens are MFMA operand A
// and weight rows operand B (v_mfma_i32_32x32x32_i8), so a lane's sixteen sums share one
// weight row (n0 + fr) and one scale per group. A step is DS MFMAs over 32 DS codes: lane
// (fr, fg) loads 8 DS bytes of its weight row and 16 DS bytes of its token row (codes
// 32 DS s + 16 DS fg .. + 16 DS - 1, one MFMA per 16 of them), so with DS = 2 (groups of 64
// or more codes) every load is 16 bytes; with DS = 1 (groups of 32) a step is one group.
// Each wave takes a contiguous range of the steps and, at the end of every group and of its
// range, converts its int32 sums and multiplies them by the group's scale into fp32 sums, as
// in the tiled grouped kernel (a group cut by a range end is folded in two parts). The
// loads of a chunk (8 KB of weights per wave, 4 KB with two token blocks, and the scale of
// each step's group) are issued before its MFMAs. Token blocks
// of eight rows that lie past M are never folded (their sums are never stored). The waves'
// fp32 sums are added in LDS in wave order; the output is bf16((sum / 16) * sa), the tiled
// kernel's epilogue.
template <int TB, int DS, bool F16>
__global__ __launch_bounds__(64 * kSmallWaves) void gemm_small_m_grouped_kernel(GemmArgs g) {
  constexpr int C = 16 / (DS * TB);                   // steps per chunk
  __shared__ float red[kSmallWaves - 1][TB][16][64];  // waves 1 .. 3's fp32 sums, [value][lane]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = (int)blockIdx.x * 32;
  const int fr = lane & 31, fg = lane >> 5;
  const int n = min(n0 + fr, g.N - 1);  // rows past the end re-read the last row (not stored)
  const uint8_t* wp = g.qw + (int64_t)n * (g.K / 2) + 8 * DS * fg;
  const uint8_t* ap[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) ap[t] = g.qa + (int64_t)min(t * 32 + fr, g.M - 1) * g.K + 16 * DS * fg;
  const int ngroups = g.K / g.group, gs = g.group / (32 * DS);  // groups, steps per group
  const int steps = g.K / (32 * DS);
  const int lo = wave * steps / kSmallWaves, nsteps = (wave + 1) * steps / kSmallWaves - lo;
  const int64_t srow = (int64_t)n * ngroups;  // this row's first group scale

  v16i_t acc[TB];
  float facc[TB][16];
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    acc[t] = v16i_t{};
#pragma unroll
    for (int e = 0; e < 16; ++e) facc[t][e] = 0.0f;
  }
  for (int j0 = 0; j0 < nsteps; j0 += C) {
    using WV = typename std::conditional<DS == 2, u32x4_g, u32x2_g>::type;
    WV w[C];
    u32x4_g a[TB][C][DS];
    float sc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      // steps past the range load its last step again (masked below)
      const int s = lo + min(j0 + c, nsteps - 1);
      w[c] = *(const WV*)(wp + (int64_t)s * 16 * DS);
      if constexpr (F16) sc[c] = (float)((const _Float16*)g.sw)[srow + s / gs];
      else sc[c] = ((const float*)g.sw)[srow + s / gs];
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int d = 0; d < DS; ++d) a[t][c][d] = *(const u32x4_g*)(ap[t] + (int64_t)s * 32 * DS + 16 * d);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = j0 + c, s = lo + j;
      const uint32_t keep = j < nsteps ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int d = 0; d < DS; ++d) {
        const v4i_t yw = widen(w[c][2 * d] & keep, w[c][2 * d + 1] & keep);
#pragma unroll
        for (int t = 0; t < TB; ++t)
          acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(order_like_widen(a[t][c][d]), yw, acc[t], 0, 0, 0);
      }
      if (j < nsteps && (s % gs == gs - 1 || j == nsteps - 1)) {  // a group's or the range's end
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (32 * t + 8 * q < g.M) {  // tokens 32 t + 8 q .. + 7
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                facc[t][4 * q + i] = fmaf((float)acc[t][4 * q + i], sc[c], facc[t][4 * q + i]);
                acc[t][4 * q + i] = 0;
              }
            }
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[wave - 1][t][e][lane] = facc[t][e];
  }
  __syncthreads();
  if (wave != 0 || n0 + fr >= g.N) return;
  // lane holds weight row n0 + fr and, per group q of four sums, token m = 32 t + 8 q + 4 fg + e
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = facc[t][e];
#pragma unroll
      for (int u = 0; u < kSmallWaves - 1; ++u) v += red[u][t][e][lane];
      const int m = t * 32 + 8 * (e / 4) + 4 * fg + (e % 4);
      if (m < g.M)
        g.out[(int64_t)m * g.N + n0 + fr] = (uint16_t)f32_to_bf16((v * 0.0625f) * load_scale(g.sa, m, g.scale_f16));
    }
}

// the few-token kernel for M <= kSmallMaxM; returns false when M is larger
template <bool A8>
static bool gemm_small_m_launch(const GemmArgs& g, hipStream_t stream) {
  if (g.M > kSmallMaxM) return false;
  const dim3 grid((uint32_t)((g.N + 15) / 16)), block(64 * kSmallWaves);
  if (g.M <= 16) hipLaunchKernelGGL((gemm_small_m_kernel<A8, 1>), grid, block, 0, stream, g);
  else if (g.M <= 32) hipLaunchKernelGGL((gemm_small_m_kernel<A8, 2>), grid, block, 0, stream, g);
  else hipLaunchKernelGGL((gemm_small_m_kernel<A8, 4>), grid, block, 0, stream, g);
  return true;
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
  if (diag_log())
    fprintf(stderr, "rbq: w4a4_gemm M=%lld N=%lld K=%lld tiles=%lld acc=%d\n", (long long)M, (long long)N,
            (long long)K, (long long)ntiles, acc != nullptr);
  if (diag_fail_launch()) return RBQ_EHIP;
  if (!gemm_small_m_launch<false>(g, stream))
    hipLaunchKernelGGL(w4a4_gemm_kernel, dim3((uint32_t)ntiles), dim3(kThreads), 0, stream, g);
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}

extern "C" rbq_status w4a8_gemm(const int8_t* qA, const void* sA, const uint8_t* qW,
                                const void* sW, rbq_dtype scale_dtype, int64_t M, int64_t N,
                                int64_t K, void* out_bf16, int32_t* acc, hipStream_t stream) {
  const rbq_status st = check_gemm(qA, sA, qW, sW, scale_dtype, M, N, K, out_bf16, acc);
  if (st != RBQ_OK || M == 0 || N == 0) return st;
  GemmArgs g{};
  g.qa = (const uint8_t*)qA; g.qw = qW; g.sa = sA; g.sw = sW;
  g.out = (uint16_t*)out_bf16;
  g.acc = acc;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.scale_f16 = scale_dtype == RBQ_F16;
  g.tiles_m = (int)((M + kBM - 1) / kBM);
  g.tiles_n = (int)((N + kBN - 1) / kBN);
  const int64_t ntiles = (int64_t)g.tiles_m * g.tiles_n;
  if (ntiles > 0x7FFFFFFF) return RBQ_ENOTSUP;
  if (diag_log())
    fprintf(stderr, "rbq: w4a8_gemm M=%lld N=%lld K=%lld tiles=%lld acc=%d\n", (long long)M, (long long)N,
            (long long)K, (long long)ntiles, acc != nullptr);
  if (diag_fail_launch()) return RBQ_EHIP;
  if (!gemm_small_m_launch<true>(g, stream))
    hipLaunchKernelGGL(w4a8_gemm_kernel, dim3((uint32_t)ntiles), dim3(kThreads), 0, stream, g);
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}

extern "C" rbq_status w4a8_gemm_grouped(const int8_t* qA, const void* sA, const uint8_t* qW,
                                        const void* sW, rbq_dtype scale_dtype, int64_t group,
                                        int64_t M, int64_t N, int64_t K, void* out_bf16,
                                        hipStream_t stream) {
  const rbq_status st = check_gemm(qA, sA, qW, sW, scale_dtype, M, N, K, out_bf16, nullptr);
  if (st != RBQ_OK) return st;
  if (group < 32 || group > K || !is_pow2(group) || K % group != 0) return RBQ_EINVAL;
  if (M == 0 || N == 0) return RBQ_OK;
  GemmArgs g{};
  g.qa = (const uint8_t*)qA; g.qw = qW; g.sa = sA; g.sw = sW;
  g.out = (uint16_t*)out_bf16;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.group = (int)group;
  g.scale_f16 = scale_dtype == RBQ_F16;
  g.tiles_m = (int)((M + kGBM - 1) / kGBM);
  g.tiles_n = (int)((N + kGBN - 1) / kGBN);
  const int64_t ntiles = (int64_t)g.tiles_m * g.tiles_n;
  if (ntiles > 0x7FFFFFFF) return RBQ_ENOTSUP;
  if (diag_log())
    fprintf(stderr, "rbq: w4a8_gemm_grouped M=%lld N=%lld K=%lld group=%lld tiles=%lld\n", (long long)M,
            (long long)N, (long long)K, (long long)group, (long long)ntiles);
  if (diag_fail_launch()) return RBQ_EHIP;
  if (M <= kSmallMaxM) {
    const dim3 sgrid((uint32_t)((N + 31) / 32)), sblock(64 * kSmallWaves);
    // instantiations: token blocks (1 or 2) x one or two MFMAs per step x fp16 or fp32 scales
    const int v = (M <= 32 ? 0 : 4) + (group == 32 ? 0 : 2) + (g.scale_f16 ? 1 : 0);
    void (*const kern[8])(GemmArgs) = {
        gemm_small_m_grouped_kernel<1, 1, false>, gemm_small_m_grouped_kernel<1, 1, true>,
        gemm_small_m_grouped_kernel<1, 2, false>, gemm_small_m_grouped_kernel<1, 2, true>,
        gemm_small_m_grouped_kernel<2, 1, false>, gemm_small_m_grouped_kernel<2, 1, true>,
        gemm_small_m_grouped_kernel<2, 2, false>, gemm_small_m_grouped_kernel<2, 2, true>};
    hipLaunchKernelGGL(kern[v], sgrid, sblock, 0, stream, g);
    return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
  }
  const dim3 grid((uint32_t)ntiles), block(kGThreads);
  const int fs = group >= 128 ? 4 : (int)(group / 32);  // sub-steps per group
  if (g.scale_f16) {
    if (fs == 1) hipLaunchKernelGGL((w4a8_gemm_grouped_kernel<1, 1>), grid, block, 0, stream, g);
    else if (fs == 2) hipLaunchKernelGGL((w4a8_gemm_grouped_kernel<1, 2>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((w4a8_gemm_grouped_kernel<1, 4>), grid, block, 0, stream, g);
  } else {
    if (fs == 1) hipLaunchKernelGGL((w4a8_gemm_grouped_kernel<0, 1>), grid, block, 0, stream, g);
    else if (fs == 2) hipLaunchKernelGGL((w4a8_gemm_grouped_kernel<0, 2>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((w4a8_gemm_grouped_kernel<0, 4>), grid, block, 0, stream, g);
  }
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}
