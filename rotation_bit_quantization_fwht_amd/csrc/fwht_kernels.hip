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

template <int K, int IN, bool ROT, bool FOURD>
__global__ __launch_bounds__((64 << KPlan<K, IN, ROT>::value.w)) void fwht_quant_kernel(KArgs a) {
  constexpr const Plan& P = KPlan<K, IN, ROT>::value;
  __shared__ float lds[lds_words(P) + (1 << P.w) + 1];
  DevCtx c;
  c.lane = threadIdx.x & 63u;
  c.wave = threadIdx.x >> 6;
  c.lds = lds;
  if constexpr (P.mfma) c.template load_hadamard_a<IN>();
  fwht_quant_wg<K, IN, ROT, FOURD>(c, a, blockIdx.x);
}

template <int K, int IN, bool ROT, bool FOURD>
static hipError_t launch_one(const KArgs& a, uint32_t grid, hipStream_t stream) {
  constexpr const Plan& P = KPlan<K, IN, ROT>::value;
  hipLaunchKernelGGL((fwht_quant_kernel<K, IN, ROT, FOURD>), dim3(grid), dim3(64u << P.w), 0,
                     stream, a);
  return hipGetLastError();
}

template <int K>
hipError_t fwht_launch(const KArgs& a, uint32_t grid, int in, bool rot, bool fourd,
                       hipStream_t s) {
  if (fourd) {
    // strided [B, H, S, D] addressing is instantiated for head_dim 64, 128 and 256
    if constexpr (K >= 6 && K <= 8) {
      if (in == IN_BF16) return launch_one<K, IN_BF16, true, true>(a, grid, s);
      return launch_one<K, IN_F16, true, true>(a, grid, s);
    } else {
      return hipErrorNotSupported;
    }
  }
  switch (in) {
    case IN_F32: return rot ? launch_one<K, IN_F32, true, false>(a, grid, s) : launch_one<K, IN_F32, false, false>(a, grid, s);
    case IN_BF16: return rot ? launch_one<K, IN_BF16, true, false>(a, grid, s) : launch_one<K, IN_BF16, false, false>(a, grid, s);
    default: return rot ? launch_one<K, IN_F16, true, false>(a, grid, s) : launch_one<K, IN_F16, false, false>(a, grid, s);
  }
}

template hipError_t fwht_launch<RBQ_K>(const KArgs&, uint32_t, int, bool, bool, hipStream_t);

}  // namespace rbq
