// gfx950 execution context for the workgroup bodies: LDS, barriers, lane shuffles,
// global memory access, the 2-term dot products that widen a packed pair of 16-bit
// values to float and apply the first radix-2 butterfly in one instruction each, and the
// 16x16x32 MFMA pair that applies the 32-point Hadamard factor to 16-bit inputs.
#pragma once

#include <hip/hip_runtime.h>

#include "fwht_engine.h"

namespace rbq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// +-1 weights of the 32-point factor in MFMA operand-A layout (see plan.h)
__constant__ HadamardA kHadamardA = make_hadamard_a();

struct DevCtx {
  uint32_t lane, wave;
  float* lds;
  u32x4_t ha[2];  // operand A of the two MFMAs for this lane (matrix plans only)

  template <int IN>
  __device__ __forceinline__ void load_hadamard_a() {
    const int f = (IN == IN_F16) ? 1 : 0;
    ha[0] = *(const u32x4_t*)&kHadamardA.w[f][0][lane][0];
    ha[1] = *(const u32x4_t*)&kHadamardA.w[f][1][lane][0];
  }

  // d = rows {j + 4m + 8 (lane / 16)} of H_32 times this wave's 16 groups of 32 inputs
  // (operand B: lane l holds elements 8 (l / 16) .. + 7 of group l mod 16)
  template <int IN>
  __device__ __forceinline__ void hadamard32(const uint32_t (&b)[4], int m, float (&d)[4]) const {
    const u32x4_t bv = {b[0], b[1], b[2], b[3]};
    const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t r;
    if constexpr (IN == IN_F16)
      r = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, ha[m]),
                                                 __builtin_bit_cast(f16x8_t, bv), z, 0, 0, 0);
    else
      r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ha[m]),
                                                  __builtin_bit_cast(bf16x8_t, bv), z, 0, 0, 0);
    d[0] = r[0]; d[1] = r[1]; d[2] = r[2]; d[3] = r[3];
  }

  // d += A B for one 16x16x32 MFMA with both operands in registers (eight 16-bit values
  // per lane each, operand layouts as in hadamard32); bf16 unless IN is IN_F16
  template <int IN>
  __device__ __forceinline__ void mfma16x16x32(const uint32_t (&a)[4], const uint32_t (&b)[4],
                                               float (&d)[4]) const {
    const u32x4_t av = {a[0], a[1], a[2], a[3]};
    const u32x4_t bv = {b[0], b[1], b[2], b[3]};
    f32x4_t cv = {d[0], d[1], d[2], d[3]};
    if constexpr (IN == IN_F16)
      cv = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av),
                                                  __builtin_bit_cast(f16x8_t, bv), cv, 0, 0, 0);
    else
      cv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                   __builtin_bit_cast(bf16x8_t, bv), cv, 0, 0, 0);
    d[0] = cv[0]; d[1] = cv[1]; d[2] = cv[2]; d[3] = cv[3];
  }

  // hides a value's origin from the optimizer (keeps a 32-bit address offset from being
  // widened and hoisted)
  __device__ __forceinline__ uint32_t opaque(uint32_t v) const {
    asm volatile("" : "+v"(v));
    return v;
  }

  // Called at the top of every block iteration: makes the lane id opaque to the compiler
  // so that per-lane address arithmetic is recomputed in each iteration instead of being
  // hoisted out of the block loop (hoisting keeps dozens of registers live across it).
  __device__ __forceinline__ void refresh_ids() { asm volatile("" : "+v"(lane)); }

  __device__ __forceinline__ void barrier() const { __syncthreads(); }
  // workgroup barrier that waits for this wave's LDS accesses only: global loads issued
  // before it (prefetches) stay in flight across it
  __device__ __forceinline__ void barrier_lds() const {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  // LDS operations of one wave execute in program order; this only keeps the
  // compiler from moving LDS accesses across the point.
  __device__ __forceinline__ void wave_sync() const { __builtin_amdgcn_wave_barrier(); }
  __device__ __forceinline__ float shfl_xor(float v, int m) const { return __shfl_xor(v, m); }
  // the same with a constant mask: masks 1 and 2 stay within a quad of lanes and take one
  // DPP move (quad permutes [1, 0, 3, 2] and [2, 3, 0, 1]) instead of an LDS permute
  template <int M>
  __device__ __forceinline__ float shfl_xor_c(float v) const {
    if constexpr (M == 1 || M == 2) {
      constexpr int ctrl = (M == 1) ? 0xB1 : 0x4E;
      return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xF, 0xF, false));
    } else {
      return __shfl_xor(v, M);
    }
  }

  template <class T>
  __device__ __forceinline__ T load(const void* p) const {
    return *(const T*)p;
  }
  template <class T>
  __device__ __forceinline__ void store(void* p, T v) const {
    *(T*)p = v;
  }
  __device__ __forceinline__ void lds_store(uint32_t i, float v) const { lds[i] = v; }
  __device__ __forceinline__ float lds_load(uint32_t i) const { return lds[i]; }
  // four consecutive words at a 16-byte aligned word index i (one 128-bit LDS access)
  __device__ __forceinline__ f32x4 lds_load4(uint32_t i) const { return *(const f32x4*)(lds + i); }
  __device__ __forceinline__ void lds_store4(uint32_t i, f32x4 v) const { *(f32x4*)(lds + i) = v; }

  // 16-bit pair (element 2j in the low half) -> two floats
  template <int IN>
  __device__ __forceinline__ void widen(uint32_t w, float& a, float& b) const {
    if constexpr (IN == IN_BF16) {
      a = bits_f32(w << 16);
      b = bits_f32(w & 0xFFFF0000u);
    } else {
      f16x2_t h = __builtin_bit_cast(f16x2_t, w);
      a = (float)h.x;
      b = (float)h.y;
    }
  }
  // same, with the radix-2 butterfly applied: (x0 + x1, x0 - x1)
  template <int IN>
  __device__ __forceinline__ void widen_butterfly(uint32_t w, float& a, float& b) const {
    if constexpr (IN == IN_BF16) {
      const bf16x2_t x = __builtin_bit_cast(bf16x2_t, w);
      a = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(bf16x2_t, 0x3F803F80u), 0.0f, false);
      b = __builtin_amdgcn_fdot2_f32_bf16(x, __builtin_bit_cast(bf16x2_t, 0xBF803F80u), 0.0f, false);
    } else {
      const f16x2_t x = __builtin_bit_cast(f16x2_t, w);
      a = __builtin_amdgcn_fdot2(x, __builtin_bit_cast(f16x2_t, 0x3C003C00u), 0.0f, false);
      b = __builtin_amdgcn_fdot2(x, __builtin_bit_cast(f16x2_t, 0xBC003C00u), 0.0f, false);
    }
  }
};

}  // namespace rbq
