// HBM streaming probe: the rate this device reaches for a given mix of reads and writes,
// shaped like the row kernels (each workgroup reads a contiguous slice, then writes a
// contiguous slice). It is the measured ceiling the HBM-bound kernels are compared with,
// beside the published peak; it computes nothing of the method.
//
// 256 threads per workgroup, 16-byte loads and stores, up to sixteen loads in flight per
// lane (all of a workgroup's slice when it is 64 KiB or less).
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

// P: 16-byte loads per lane per batch, all issued before any is used (a row kernel loads
// its whole row that way)
template <int P>
__global__ __launch_bounds__(kProbeThreads) void hbm_probe_kernel(const char* src, int64_t rd, char* dst,
                                                                  int64_t wr, uint32_t marker) {
  const int64_t b = blockIdx.x;
  const probe_u32x4* s = (const probe_u32x4*)(src + b * rd) + threadIdx.x;
  uint32_t fold = 0;
  const int64_t passes = rd / kProbeChunk;
  for (int64_t p = 0; p < passes; p += P) {
    probe_u32x4 v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) v[i] = s[(p + i) * kProbeThreads];
#pragma unroll
    for (int i = 0; i < P; ++i) fold ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
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
  // as many loads in flight per lane as the block's slice allows, up to 16
  const int64_t passes = read_bytes_per_block / kProbeChunk;
  const dim3 grid((uint32_t)blocks), block(kProbeThreads);
  const uint32_t marker = 0x9E3779B9u;
  const char* sp = (const char*)src;
  char* dp = (char*)dst;
  const int64_t rd = read_bytes_per_block, wr = write_bytes_per_block;
  if (passes % 16 == 0 && passes > 0) hipLaunchKernelGGL(hbm_probe_kernel<16>, grid, block, 0, stream, sp, rd, dp, wr, marker);
  else if (passes % 8 == 0 && passes > 0) hipLaunchKernelGGL(hbm_probe_kernel<8>, grid, block, 0, stream, sp, rd, dp, wr, marker);
  else if (passes % 4 == 0 && passes > 0) hipLaunchKernelGGL(hbm_probe_kernel<4>, grid, block, 0, stream, sp, rd, dp, wr, marker);
  else if (passes % 2 == 0 && passes > 0) hipLaunchKernelGGL(hbm_probe_kernel<2>, grid, block, 0, stream, sp, rd, dp, wr, marker);
  else hipLaunchKernelGGL(hbm_probe_kernel<1>, grid, block, 0, stream, sp, rd, dp, wr, marker);
  return hipGetLastError() == hipSuccess ? RBQ_OK : RBQ_EHIP;
}
