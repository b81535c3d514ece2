// gfx950 execution context for the workgroup bodies: LDS, barriers, lane shuffles,
// global memory access and the 2-term dot products that widen a packed pair of 16-bit
// values to float and apply the first radix-2 butterfly in one instruction each.
#pragma once

#include <hip/hip_runtime.h>

#include "fwht_engine.h"

namespace rbq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

struct DevCtx {
  uint32_t lane, wave;
  float* lds;

  __device__ __forceinline__ void barrier() const { __syncthreads(); }
  // LDS operations of one wave execute in program order; this only keeps the
  // compiler from moving LDS accesses across the point.
  __device__ __forceinline__ void wave_sync() const { __builtin_amdgcn_wave_barrier(); }
  __device__ __forceinline__ float shfl_xor(float v, int m) const { return __shfl_xor(v, m); }

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
