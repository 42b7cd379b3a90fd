// Streaming-read diagnostic: the same non-temporal 128-bit loads that the
// decode kernels use to stream the packed cache, over a plain buffer.  Gives
// the achievable read bandwidth of the device and a known-size reference
// for the HBM byte counters.
#include "device_common.h"

namespace tq {
namespace {

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4s* __restrict__ src, size_t n, uint32_t* sink) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (; i < n; i += stride) {
    const u32x4s v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t s[256];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int k = 0; k < 256; ++k) a ^= s[k];
    sink[blockIdx.x] = a;
  }
}

}  // namespace

int stream_read_blocks() { return 2048; }

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(stream_read_blocks()), dim3(256), 0, s,
                     reinterpret_cast<const u32x4s*>(src), bytes / 16, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace tq
