// Streaming-read probe: the rate at which this device streams a buffer from
// HBM with plain 16-byte loads, the ceiling the HBM-bound decode kernels are
// compared with (besides the 8 TB/s of the specification).  Diagnostics only;
// no decode path uses it.
#include "common.hpp"
#include "internal.hpp"

namespace dattn {
namespace {

constexpr int kProbeThreads = 256;

// Workgroup g streams its own contiguous range of the buffer; each thread
// keeps U independent 16-byte loads in flight per step (a wave: U KB).
template <int U>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* src, size_t n16,
                                                                    uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t begin = (size_t)blockIdx.x * per;
  const size_t end = begin + per < n16 ? begin + per : n16;
  constexpr size_t kStepVecs = (size_t)U * kProbeThreads;
  uint32_t acc = 0;
  size_t i = begin + threadIdx.x;
  for (; i + (U - 1) * kProbeThreads < end; i += kStepVecs) {
    uint4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = load_stream(src + i + j * kProbeThreads);
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < end; i += kProbeThreads) {
    const uint4 v = load_stream(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the loads must not be optimised away; the store almost never happens
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, int depth,
                              hipStream_t s) {
  const uint4* p = (const uint4*)src;
  switch (depth) {
    case 4: launch_kernel(stream_read_kernel<4>, dim3(grid), dim3(kProbeThreads), s, p, bytes / 16, sink); break;
    case 8: launch_kernel(stream_read_kernel<8>, dim3(grid), dim3(kProbeThreads), s, p, bytes / 16, sink); break;
    case 16: launch_kernel(stream_read_kernel<16>, dim3(grid), dim3(kProbeThreads), s, p, bytes / 16, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dattn
