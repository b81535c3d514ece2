// Kernel instantiations of the fused Hadamard + INT4 quantizer for one row length
// n = 2^RBQ_K (the build compiles this file once per RBQ_K, in parallel).
#include <hip/hip_runtime.h>

#include "devctx.h"

#ifndef RBQ_K
#error "compile with -DRBQ_K=<log2 n>"
#endif

namespace rbq {

template <int K, int IN, bool ROT>
using KPlan = PlanOf<K, use_matrix_plan(K, IN, ROT)>;

#ifndef RBQ_WAVES_PER_EU
#define RBQ_WAVES_PER_EU 4
#endif
#ifndef RBQ_RESIDENT_GRID
#define RBQ_RESIDENT_GRID 0
#endif

// at least RBQ_WAVES_PER_EU waves per SIMD: enough resident workgroups to overlap one
// block's loads with another's arithmetic. The variants that also write rotated values
// keep more live registers; they get one wave less rather than spilling. Plans with 32
// values per lane aim at 8 waves (64 registers), 6 when they also write rotated values.
// The RoPE variants hold each load's cos/sin values as well and get 4 waves (2 for rows of
// 64 and 256, whose loads carry twice the table values per lane).
template <int K, int IN, bool ROT>
constexpr int fwht_waves_per_eu(bool fast, bool rope) {
  if (rope) return K == 7 ? 4 : 2;
  if (KPlan<K, IN, ROT>::value.e == 5) return fast ? 8 : 6;
  return fast ? RBQ_WAVES_PER_EU : RBQ_WAVES_PER_EU - 1;
}

// CACHE: codes and scales rows may go to a per-head cache (TensorArgs::out_cap)
template <int K, int IN, bool ROT, bool FOURD, bool FAST, bool ROPE, bool CACHE>
__global__ __launch_bounds__((64 << KPlan<K, IN, ROT>::value.w)) __attribute__((amdgpu_waves_per_eu(fwht_waves_per_eu<K, IN, ROT>(FAST, ROPE))))
void fwht_quant_kernel(KArgs a) {
  constexpr const Plan& P = KPlan<K, IN, ROT>::value;
  __shared__ float lds[lds_words(P) + (1 << P.w) + 1];
  DevCtx c;
  c.lane = threadIdx.x & 63u;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers
  c.lds = lds;
  if constexpr (P.mfma) c.template load_hadamard_a<IN>();
  fwht_quant_persistent<K, IN, ROT, FOURD, FAST, ROPE, CACHE>(c, a, blockIdx.x, gridDim.x);
}

// Workgroups loop over the row blocks (see fwht_quant_persistent); the grid holds as many
// workgroups as fit on the device at once, or fewer when there are fewer blocks.
template <int K, int IN, bool ROT, bool FOURD, bool FAST = false, bool ROPE = false, bool CACHE = false>
static hipError_t launch_one(const KArgs& a, hipStream_t stream) {
  constexpr const Plan& P = KPlan<K, IN, ROT>::value;
  constexpr int threads = 64 << P.w;
  static const int per_cu = [] {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, fwht_quant_kernel<K, IN, ROT, FOURD, FAST, ROPE, CACHE>, threads, 0) !=
            hipSuccess || o < 1)
      o = 1;
    return o;
  }();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return hipErrorInvalidDevice;
  // one workgroup per block, or (RBQ_RESIDENT_GRID) only as many as are resident at once
  const uint64_t cap = RBQ_RESIDENT_GRID ? (uint64_t)per_cu * (uint64_t)cus : 0xFFFFFFFFull;
  const uint32_t grid = (uint32_t)(a.nblocks < cap ? a.nblocks : cap);
  hipLaunchKernelGGL((fwht_quant_kernel<K, IN, ROT, FOURD, FAST, ROPE, CACHE>), dim3(grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

// fast: packed codes and scales are the only outputs (no rotated rows, no int8 codes)
// rope: RoPE before the transform (16-bit Q/K of head_dim 64, 128 or 256)
// cache: 16-bit rows of head_dim 64, 128 or 256 addressed as [B, H, S, D], codes and
//        scales possibly written to a per-head cache; the blocks from a.blocks1 on quantize
//        the rows of a.tv as they are
template <int K>
hipError_t fwht_launch(const KArgs& a, int in, bool rot, bool fourd, bool fast, bool rope, bool cache,
                       hipStream_t s) {
  if (cache) {
    if constexpr (K >= 6 && K <= 8) {
      if (in == IN_F32 || !fourd || fast || !rot) return hipErrorNotSupported;
      if (in == IN_BF16)
        return rope ? launch_one<K, IN_BF16, true, true, false, true, true>(a, s)
                    : launch_one<K, IN_BF16, true, true, false, false, true>(a, s);
      return rope ? launch_one<K, IN_F16, true, true, false, true, true>(a, s)
                  : launch_one<K, IN_F16, true, true, false, false, true>(a, s);
    } else {
      return hipErrorNotSupported;
    }
  }
  if (rope) {
    if constexpr (K >= 6 && K <= 8) {
      if (!rot || in == IN_F32) return hipErrorNotSupported;
      if (fourd) {
        if (in == IN_BF16)
          return fast ? launch_one<K, IN_BF16, true, true, true, true>(a, s) : launch_one<K, IN_BF16, true, true, false, true>(a, s);
        return fast ? launch_one<K, IN_F16, true, true, true, true>(a, s) : launch_one<K, IN_F16, true, true, false, true>(a, s);
      }
      if (in == IN_BF16)
        return fast ? launch_one<K, IN_BF16, true, false, true, true>(a, s) : launch_one<K, IN_BF16, true, false, false, true>(a, s);
      return fast ? launch_one<K, IN_F16, true, false, true, true>(a, s) : launch_one<K, IN_F16, true, false, false, true>(a, s);
    } else {
      return hipErrorNotSupported;
    }
  }
  if (fourd) {
    // strided [B, H, S, D] addressing is instantiated for head_dim 64, 128 and 256
    if constexpr (K >= 6 && K <= 8) {
      if (in == IN_BF16)
        return fast ? launch_one<K, IN_BF16, true, true, true>(a, s) : launch_one<K, IN_BF16, true, true>(a, s);
      return fast ? launch_one<K, IN_F16, true, true, true>(a, s) : launch_one<K, IN_F16, true, true>(a, s);
    } else {
      return hipErrorNotSupported;
    }
  }
  switch (in) {
    case IN_F32:
      return rot ? launch_one<K, IN_F32, true, false>(a, s) : launch_one<K, IN_F32, false, false>(a, s);
    case IN_BF16:
      if (!rot) return launch_one<K, IN_BF16, false, false>(a, s);
      return fast ? launch_one<K, IN_BF16, true, false, true>(a, s) : launch_one<K, IN_BF16, true, false>(a, s);
    default:
      if (!rot) return launch_one<K, IN_F16, false, false>(a, s);
      return fast ? launch_one<K, IN_F16, true, false, true>(a, s) : launch_one<K, IN_F16, true, false>(a, s);
  }
}

template hipError_t fwht_launch<RBQ_K>(const KArgs&, int, bool, bool, bool, bool, bool, hipStream_t);

}  // namespace rbq
