// HIP kernels and C-ABI entry points of the rotation + INT4 quantizer for row lengths
// that are not powers of two (n = m * p, H_m (x) H_p with a Paley or Goethals-Seidel factor; the body is in
// kron_engine.h, the choice of m in kron_factor.h). Powers of two go to the
// power-of-two path of hadamard_quant_int4.
#include <hip/hip_runtime.h>

#include "../../include/rbq.h"
#include "devctx.h"
#include "diag.h"
#include "kron_engine.h"
#include "kron_factor.h"
#include "validate.h"

namespace rbq {

// LW: LDS words of the variant (32 KiB, 80 KiB or 160 KiB), the smallest that holds the
// row buffer and the operand table; smaller variants keep more workgroups per CU.
// KS 1: rows with one K block of the MFMA (m <= 32), KS 0: two to five (m <= 160), KS 2:
// six (m <= 192), KS 3: seven and eight (m <= 256); each has its own wave count and
// register budget (for m <= 32, 8 waves at up to 128 VGPRs; otherwise up to 256: 4 waves,
// or, for six K blocks, 8 in the one workgroup per CU that their LDS allows).
template <int IN, uint32_t LW, int KS>
__global__ __launch_bounds__((64 * kron_body_waves<IN, KS>()))
__attribute__((amdgpu_waves_per_eu((KS == 1 && kron_body_waves<IN, KS>() == 8u) ? 4 : 2)))
void kron_quant_kernel(KronArgs a) {
  __shared__ float lds[LW];
  DevCtx c;
  c.lane = threadIdx.x & 63u;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.lds = lds;
  kron_quant_body<IN, KS>(c, a, blockIdx.x, gridDim.x);
}

// Workgroups loop over rows: the grid holds as many as are resident at once (each one
// prefetches its next row's first operands while it finishes the current row), or one
// per row when there are fewer rows.
template <int IN, uint32_t LW, int KS>
static hipError_t kron_launch_lw(const KronArgs& a, hipStream_t s) {
  constexpr int NT = 64 * (int)kron_body_waves<IN, KS>();
  static const int per_cu = [] {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kron_quant_kernel<IN, LW, KS>, NT, 0) != hipSuccess ||
        o < 1)
      o = 1;
    return o;
  }();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return hipErrorInvalidDevice;
  const int64_t cap = (int64_t)per_cu * cus;
  const uint32_t grid = (uint32_t)(a.rows < cap ? a.rows : cap);
  if (diag_log()) fprintf(stderr, "rbq: hadamard_kron_quant lds_words=%u grid=%u threads=%d\n", LW, grid, NT);
  hipLaunchKernelGGL((kron_quant_kernel<IN, LW, KS>), dim3(grid), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int IN, int KS>
static hipError_t kron_launch_ks(const KronArgs& a, uint32_t words, hipStream_t s) {
  if (words <= 8192u) return kron_launch_lw<IN, 8192u, KS>(a, s);
  if (words <= 20480u) return kron_launch_lw<IN, 20480u, KS>(a, s);
  return kron_launch_lw<IN, 40960u, KS>(a, s);
}

template <int IN>
static hipError_t kron_launch_in(const KronArgs& a, uint32_t words, hipStream_t s) {
  if (a.m <= 32u) return kron_launch_ks<IN, 1>(a, words, s);
  if (a.m <= 160u) return kron_launch_ks<IN, 0>(a, words, s);
  // orders above 160: the operand table alone takes more than 80 KiB
  if (a.m <= 192u) return kron_launch_lw<IN, 40960u, 2>(a, s);
  return kron_launch_lw<IN, 40960u, 3>(a, s);
}

}  // namespace rbq

using namespace rbq;

extern "C" rbq_status rbq_kron_factor(int64_t n, int64_t* m) {
  if (!m || n < 1) return RBQ_EINVAL;
  const KronFactor f = kron_factor(n);
  if (f.m == 0) return RBQ_ENOTSUP;
  *m = f.m;
  return RBQ_OK;
}

extern "C" rbq_status hadamard_kron_quant_int4(const void* x, rbq_dtype x_dtype, int64_t n,
                                               int64_t tokens, int64_t x_row_stride, void* codes,
                                               void* scales, rbq_dtype scale_dtype, float* rotated,
                                               unsigned flags, hipStream_t stream) {
  if (flags & ~(unsigned)RBQ_PACKED) return RBQ_EINVAL;
  if (!valid_in_dtype(x_dtype) || !valid_scale_dtype(scale_dtype)) return RBQ_EINVAL;
  if (n < 2 || n > 32768 || tokens < 0) return RBQ_EINVAL;
  if (is_pow2(n))
    return hadamard_quant_int4(x, x_dtype, n, tokens, x_row_stride, codes, scales, scale_dtype,
                               rotated, flags, stream);
  KronArgs a{};
  const uint32_t words = kron_setup(n, a);
  if (words == 0) return RBQ_ENOTSUP;
  if (tokens == 0) return RBQ_OK;
  if (!x || !codes || !scales) return RBQ_EINVAL;
  const int64_t esz = dtype_size(x_dtype);
  if (x_row_stride < n || !aligned(x, 16) || ((x_row_stride * esz) % 16) != 0) return RBQ_EINVAL;
  if (!aligned(codes, 16) || !aligned(scales, (uint64_t)dtype_size(scale_dtype))) return RBQ_EINVAL;
  if (rotated && !aligned(rotated, 16)) return RBQ_EINVAL;
  a.x = x;
  a.row_stride = x_row_stride;
  a.rows = tokens;
  a.codes = codes;
  a.scales = scales;
  a.rot32 = rotated;
  a.opts = ((flags & RBQ_PACKED) ? OPT_PACKED : 0u) | (scale_dtype == RBQ_F16 ? OPT_SCALE_F16 : 0u);
  if (diag_log())
    fprintf(stderr, "rbq: hadamard_kron_quant n=%lld m=%u p=%u paley=%u q=%u tokens=%lld dtype=%d packed=%d\n",
            (long long)n, a.m, 1u << a.p_log, a.paley, a.q, (long long)tokens, (int)x_dtype,
            (flags & RBQ_PACKED) != 0);
  if (diag_fail_launch()) return RBQ_EHIP;
  hipError_t e;
  switch (x_dtype) {
    case RBQ_F32: e = kron_launch_in<IN_F32>(a, words, stream); break;
    case RBQ_BF16: e = kron_launch_in<IN_BF16>(a, words, stream); break;
    default: e = kron_launch_in<IN_F16>(a, words, stream); break;
  }
  return e == hipSuccess ? RBQ_OK : RBQ_EHIP;
}
