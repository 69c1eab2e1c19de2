// Streaming-read reference kernel: the HBM read rate that a kernel which
// reads its input exactly once can reach on this device.  It is the
// achievable ceiling that the logits pass (one read of every drafter logit)
// is compared against, beside the nominal peak.
//
// Layout of the work: a grid of kBlocksPerCU workgroups per compute unit,
// 256 threads each, striding over the buffer in 16-byte nontemporal loads
// (consecutive lanes read consecutive 16-byte words, so each wave reads one
// 1 KiB run per step).  Every word is folded into an XOR checksum so that the
// loads cannot be dropped and the result can be checked.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfd_device.hpp"
#include "mfd_launch.hpp"

namespace mfd {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kCUs = 256;
constexpr int kBlocksPerCU = 8;

__global__ void __launch_bounds__(kReadThreads) stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  for (size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
  __shared__ uint32_t part[kReadThreads / kWave];
  if (lane_id() == 0) part[wave_id()] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < kReadThreads / kWave; ++w) a ^= part[w];
    atomicXor(sink, a);
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t want = (n16 + kReadThreads - 1) / kReadThreads;
  const int grid = (int)(want < (size_t)kCUs * kBlocksPerCU ? want : (size_t)kCUs * kBlocksPerCU);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace mfd
