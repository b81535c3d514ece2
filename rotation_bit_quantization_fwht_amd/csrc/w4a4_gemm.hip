// W4A4 GEMM entry point (kernel to follow): argument validation only for now.
#include <hip/hip_runtime.h>

#include "../../include/rbq.h"
#include "validate.h"

extern "C" rbq_status w4a4_gemm(const uint8_t* qA, const void* sA, const uint8_t* qW,
                                const void* sW, rbq_dtype scale_dtype, int64_t M, int64_t N,
                                int64_t K, void* out_bf16, int32_t* acc, hipStream_t stream) {
  (void)stream;
  const rbq_status st = rbq::check_gemm(qA, sA, qW, sW, scale_dtype, M, N, K, out_bf16, acc);
  if (st != RBQ_OK || M == 0 || N == 0) return st;
  return RBQ_ENOTSUP;
}
