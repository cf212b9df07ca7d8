// Read-rate reference: a kernel that does nothing but stream a buffer from
// HBM, with the access pattern the decode kernels use for their tiles
// (16-byte non-temporal loads, one contiguous range per workgroup, one
// workgroup per compute unit, 32 KB in flight per compute unit).  Its time
// over the same byte count as a decode call is a practical read reference
// for the attention kernels, next to the published HBM peak (a reference,
// not a bound).  Each thread folds its words with XOR into one word of the sink, so
// the loads cannot be dropped; the XOR of the whole sink equals the XOR of
// every 32-bit word of the buffer.
#include <hip/hip_runtime.h>

#include "device_common.h"

namespace mfa {
namespace {

constexpr int kThreads = 512;
constexpr int kInFlight = 4;   // 16-byte loads per thread between waits

__global__ void __launch_bounds__(kThreads) stream_read_kernel(const intx4* __restrict__ src, int64_t n16,
                                                               int32_t* __restrict__ sink) {
  const int64_t w = blockIdx.x, nw = gridDim.x;
  const int64_t lo = w * n16 / nw, hi = (w + 1) * n16 / nw;
  intx4 acc = {0, 0, 0, 0};
  for (int64_t i = lo + threadIdx.x; i < hi; i += (int64_t)kThreads * kInFlight) {
    intx4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const int64_t idx = i + (int64_t)k * kThreads;
      v[k] = __builtin_nontemporal_load(src + (idx < hi ? idx : hi - 1));   // clamped, then masked
      if (idx >= hi) v[k] = intx4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k];
  }
  sink[w * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

int stream_read_threads() { return kThreads; }

hipError_t launch_stream_read(const void* src, int64_t bytes, int32_t* sink, int workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                     static_cast<const intx4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace mfa
