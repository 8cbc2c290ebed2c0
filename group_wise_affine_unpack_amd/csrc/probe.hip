// Streaming-read probe: the achievable HBM read rate on this device, the
// denominator measured beside the published peak.  Each thread reads
// 16-byte pieces with non-temporal buffer loads, grid-strided so that a
// wave's load covers whole 1 KiB and every CU has several waves in flight,
// and folds them into one word it writes to `sink` (so no load is dead).
// The grid is a multiple of the CU count; no result other than the sink.
#include "common.h"

namespace qaff {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, long n16,
                                                          uint32_t* __restrict__ sink) {
  const long tid = (long)blockIdx.x * 256 + threadIdx.x, stride = (long)gridDim.x * 256;
  u32x4_t a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
  long i = tid;
  // two loads in flight per iteration
  for (; i + stride < n16; i += 2 * stride) {
    a ^= __builtin_nontemporal_load(src + i);
    b ^= __builtin_nontemporal_load(src + i + stride);
  }
  if (i < n16) a ^= __builtin_nontemporal_load(src + i);
  a ^= b;
  sink[tid] = a.x ^ a.y ^ a.z ^ a.w;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s, (const u32x4_t*)src, (long)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace qaff
