// Group-wise symmetric INT4 quantization of rows already in the rotated basis: one absmax
// scale per run of G consecutive elements ("SpinQuant, when rotations are worth learning":
// the ExecuTorch export quantizes 4-bit weights in groups of 256 or 32 input channels; the
// step-size equation of "SpinQuant Guide: Learned Rotations for 4-Bit LLMs" per group).
//
// Each lane takes E consecutive elements (E = max(8, G / 64)), so a group spans G / E <= 64
// lanes of one wave: the group maximum is a shuffle reduction over those lanes, and the
// lane's codes are one contiguous run of E / 2 packed bytes. The rounding decision is the
// exact round-half-even of y / s_stored (ties are common when the input is quantized as
// is).
#include <hip/hip_runtime.h>

#include "../../include/rbq.h"
#include "diag.h"
#include "fwht_engine.h"
#include "validate.h"

namespace rbq {

struct GroupArgs {
  const void* y;
  int64_t row_stride;  // elements
  int64_t rows;
  void* codes;
  void* scales;
  uint32_t K, group, lanes_log;  // lanes per group = 2^lanes_log
  uint32_t packed, scale_f16;
};

template <int IN, int E>
__global__ __launch_bounds__(256) void group_quant_kernel(GroupArgs a) {
  constexpr int ESZ = (IN == IN_F32) ? 4 : 2;
  const uint32_t chunks_per_row = a.K / E;
  const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = chunk < a.rows * (int64_t)chunks_per_row;
  const int64_t row = valid ? chunk / chunks_per_row : 0;
  const uint32_t c = valid ? (uint32_t)(chunk - row * chunks_per_row) : 0;
  const uint32_t e0 = c * E;

  float v[E];
  const char* src = (const char*)a.y + (row * a.row_stride + e0) * ESZ;
  static_for<0, E * ESZ / 16>([&](auto Q) {
    const u32x4 w = valid ? *(const u32x4*)(src + 16 * Q.value) : u32x4{0u, 0u, 0u, 0u};
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    if constexpr (IN == IN_F32) {
      static_for<0, 4>([&](auto I) { v[4 * Q.value + I.value] = bits_f32(ws[I.value]); });
    } else {
      static_for<0, 4>([&](auto I) {
        const uint32_t lo = ws[I.value] & 0xFFFFu, hi = ws[I.value] >> 16;
        v[8 * Q.value + 2 * I.value] = (IN == IN_F16) ? f16_to_f32(lo) : bf16_to_f32(lo);
        v[8 * Q.value + 2 * I.value + 1] = (IN == IN_F16) ? f16_to_f32(hi) : bf16_to_f32(hi);
      });
    }
  });

  // group maximum across the 2^lanes_log >= 4 lanes of the group (groups never straddle
  // waves): within a row of sixteen lanes by DPP moves (quad swaps, then the quads of each
  // half and the halves of the row by mirrors), across rows by lane permutes; every lane
  // is active here
  float mx = 0.0f;
  static_for<0, E>([&](auto I) { mx = fmaxf(mx, fabsf(v[I.value])); });
  auto dpp = [](float x, auto CTRL) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), decltype(CTRL)::value,
                                                                 0xF, 0xF, false));
  };
  mx = fmaxf(mx, dpp(mx, IC<0xB1>{}));                    // quad_perm [1, 0, 3, 2]
  mx = fmaxf(mx, dpp(mx, IC<0x4E>{}));                    // quad_perm [2, 3, 0, 1]
  if (a.lanes_log >= 3) mx = fmaxf(mx, dpp(mx, IC<0x141>{}));  // row_half_mirror
  if (a.lanes_log >= 4) mx = fmaxf(mx, dpp(mx, IC<0x140>{}));  // row_mirror
  if (a.lanes_log >= 5) mx = fmaxf(mx, __shfl_xor(mx, 16));
  if (a.lanes_log >= 6) mx = fmaxf(mx, __shfl_xor(mx, 32));

  float s = fmaxf(mx / 7.0f, 1e-8f);
  uint32_t h16 = 0;
  if (a.scale_f16) { h16 = f32_to_f16(s); s = f16_to_f32(h16); }
  const float mk = (s == 0.0f) ? 0.0f : 1.0f / s;
  if (!valid) return;
  if ((c & ((1u << a.lanes_log) - 1u)) == 0) {
    const int64_t si = row * (int64_t)(a.K / a.group) + e0 / a.group;
    if (a.scale_f16) ((uint16_t*)a.scales)[si] = (uint16_t)h16;
    else ((float*)a.scales)[si] = s;
  }
  auto code = [&](float u) {
    float q = round_quotient_exact(u, mk, s) + kMagic;
    q = fminf(fmaxf(q, kMagic - 8.0f), kMagic + 7.0f);
    return f32_bits(q);
  };
  if (a.packed) {
    uint32_t w[E / 8];
    static_for<0, E / 8>([&](auto D) {
      uint32_t acc = 0;
      static_for<0, 8>([&](auto I) { acc = alignbit(code(v[8 * D.value + I.value]), acc, 4); });
      w[D.value] = acc;
    });
    uint8_t* dst = (uint8_t*)a.codes + row * (int64_t)(a.K / 2) + e0 / 2;
    if constexpr (E == 8) {
      *(uint32_t*)dst = w[0];
    } else if constexpr (E == 16) {
      *(u32x2*)dst = u32x2{w[0], w[1]};
    } else {
      static_for<0, E / 32>([&](auto Q) {
        *(u32x4*)(dst + 16 * Q.value) = u32x4{w[4 * Q.value], w[4 * Q.value + 1], w[4 * Q.value + 2], w[4 * Q.value + 3]};
      });
    }
  } else {
    uint32_t w[E / 4];
    static_for<0, E / 4>([&](auto D) {
      uint32_t acc = 0;
      static_for<0, 4>([&](auto I) { acc = alignbit(code(v[4 * D.value + I.value]), acc, 8); });
      w[D.value] = acc;
    });
    uint8_t* dst = (uint8_t*)a.codes + row * (int64_t)a.K + e0;
    static_for<0, E / 16>([&](auto Q) {
      *(u32x4*)(dst + 16 * Q.value) = u32x4{w[4 * Q.value], w[4 * Q.value + 1], w[4 * Q.value + 2], w[4 * Q.value + 3]};
    });
    if constexpr (E == 8) *(u32x2*)dst = u32x2{w[0], w[1]};
  }
}

template <int IN>
static hipError_t group_launch(const GroupArgs& a, uint32_t E, uint32_t blocks, hipStream_t s) {
  switch (E) {
    case 8: hipLaunchKernelGGL((group_quant_kernel<IN, 8>), dim3(blocks), dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((group_quant_kernel<IN, 16>), dim3(blocks), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((group_quant_kernel<IN, 32>), dim3(blocks), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((group_quant_kernel<IN, 64>), dim3(blocks), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace rbq

using namespace rbq;

extern "C" rbq_status quantize_groups_int4(const void* y, rbq_dtype dtype, int64_t K, int64_t rows,
                                           int64_t y_row_stride, int64_t group, void* codes, void* scales,
                                           rbq_dtype scale_dtype, unsigned flags, hipStream_t stream) {
  if (flags & ~(unsigned)RBQ_PACKED) return RBQ_EINVAL;
  if (!valid_in_dtype(dtype) || !valid_scale_dtype(scale_dtype)) return RBQ_EINVAL;
  if (rows < 0 || K < 32 || K > 65536 || group < 32 || group > 4096 || group > K || !is_pow2(group) ||
      K % group != 0)
    return RBQ_EINVAL;
  if (rows == 0) return RBQ_OK;
  if (!y || !codes || !scales) return RBQ_EINVAL;
  const int64_t esz = dtype_size(dtype);
  if (y_row_stride < K || !aligned(y, 16) || (y_row_stride * esz) % 16 != 0) return RBQ_EINVAL;
  if (!aligned(codes, 16) || !aligned(scales, (uint64_t)dtype_size(scale_dtype))) return RBQ_EINVAL;
  const uint32_t E = group / 64 > 8 ? (uint32_t)(group / 64) : 8u;
  const int64_t chunks = rows * (K / E);
  if ((chunks + 255) / 256 > 0x7FFFFFFF) return RBQ_EINVAL;
  GroupArgs a{};
  a.y = y;
  a.row_stride = y_row_stride;
  a.rows = rows;
  a.codes = codes;
  a.scales = scales;
  a.K = (uint32_t)K;
  a.group = (uint32_t)group;
  a.lanes_log = (uint32_t)ilog2(group / E);
  a.packed = (flags & RBQ_PACKED) != 0;
  a.scale_f16 = scale_dtype == RBQ_F16;
  const uint32_t blocks = (uint32_t)((chunks + 255) / 256);
  if (diag_log())
    fprintf(stderr, "rbq: quantize_groups_int4 K=%lld rows=%lld group=%lld dtype=%d elems_per_lane=%u blocks=%u\n",
            (long long)K, (long long)rows, (long long)group, (int)dtype, E, blocks);
  if (diag_fail_launch()) return RBQ_EHIP;
  hipError_t e;
  switch (dtype) {
    case RBQ_F32: e = group_launch<IN_F32>(a, E, blocks, stream); break;
    case RBQ_BF16: e = group_launch<IN_BF16>(a, E, blocks, stream); break;
    default: e = group_launch<IN_F16>(a, E, blocks, stream); break;
  }
  return e == hipSuccess ? RBQ_OK : RBQ_EHIP;
}
