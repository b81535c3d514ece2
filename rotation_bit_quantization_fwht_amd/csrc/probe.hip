// HBM streaming probe: the rate this device reaches for a given mix of reads and writes,
// shaped like the row kernels (each workgroup reads a contiguous slice, then writes a
// contiguous slice). It is the measured ceiling the HBM-bound kernels are compared with,
// beside the published peak; it computes nothing of the method.
//
// 256 threads per workgroup, 16-byte loads and stores, four loads in flight per lane.
// The loaded words are folded with xor into one value that every store writes, so the
// loads cannot be dropped; with no write slice, one word per workgroup is written only if
// the fold hits a value the caller's fill never produces.
#include <hip/hip_runtime.h>

#include "../../include/rbq.h"
#include "diag.h"

namespace rbq {

typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeChunk = kProbeThreads * 16;  // bytes one pass of the workgroup moves

__global__ __launch_bounds__(kProbeThreads) void hbm_probe_kernel(const char* src, int64_t rd, char* dst,
                                                                  int64_t wr, uint32_t marker) {
  const int64_t b = blockIdx.x;
  const probe_u32x4* s = (const probe_u32x4*)(src + b * rd) + threadIdx.x;
  uint32_t fold = 0;
  const int64_t passes = rd / kProbeChunk;
  int64_t p = 0;
  for (; p + 4 <= passes; p += 4) {
    probe_u32x4 v0 = s[(p + 0) * kProbeThreads];
    probe_u32x4 v1 = s[(p + 1) * kProbeThreads];
    probe_u32x4 v2 = s[(p + 2) * kProbeThreads];
    probe_u32x4 v3 = s[(p + 3) * kProbeThreads];
    probe_u32x4 x = v0 ^ v1 ^ v2 ^ v3;
    fold ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  for (; p < passes; ++p) {
    probe_u32x4 v = s[p * kProbeThreads];
    fold ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (wr == 0) {
    if (fold == marker) *(uint32_t*)(dst + b * 16 + (threadIdx.x & 3) * 4) = fold;
    return;
  }
  probe_u32x4* d = (probe_u32x4*)(dst + b * wr) + threadIdx.x;
  const probe_u32x4 o = {fold, fold, fold, fold};
  const int64_t wpasses = wr / kProbeChunk;
  for (int64_t q = 0; q < wpasses; ++q) d[q * kProbeThreads] = o;
}

}  // namespace rbq

using namespace rbq;

extern "C" rbq_status rbq_hbm_probe(const void* src, int64_t read_bytes_per_block, void* dst,
                                    int64_t write_bytes_per_block, int64_t blocks, hipStream_t stream) {
  if (blocks < 0 || read_bytes_per_block < 0 || write_bytes_per_block < 0) return RBQ_EINVAL;
  if (read_bytes_per_block % kProbeChunk || write_bytes_per_block % kProbeChunk) return RBQ_EINVAL;
  if (read_bytes_per_block == 0 && write_bytes_per_block == 0) return RBQ_EINVAL;
  if (blocks == 0) return RBQ_OK;
  if (blocks > 0x7FFFFFFF) return RBQ_EINVAL;
  if (dst == nullptr || (read_bytes_per_block > 0 && src == nullptr)) return RBQ_EINVAL;
  if (((uintptr_t)src | (uintptr_t)dst) & 15u) return RBQ_EINVAL;
  if (diag_log())
    fprintf(stderr, "rbq: hbm_probe read=%lld write=%lld blocks=%lld\n", (long long)read_bytes_per_block,
            (long long)write_bytes_per_block, (long long)blocks);
  if (diag_fail_launch()) return RBQ_EHIP;
  hipLaunchKernelGGL(hbm_probe_kernel, dim3((uint32_t)blocks), dim3(kProbeThreads), 0, stream, (const char*)src,
                     read_bytes_per_block, (char*)dst, write_bytes_per_block, 0x9E3779B9u);
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}
