// Streaming diagnostics.
//   * stream read: the same non-temporal 128-bit loads that the decode
//     kernels use to stream the packed cache, over a plain buffer.  Gives the
//     achievable read bandwidth of the device and a known-size reference for
//     the HBM byte counters.
//   * stream read-write: the write side's memory traffic with no arithmetic.
//     A wave takes 16 rows; lane (g, tau) reads 16-byte chunks g, g + 4, ...
//     of row tau and writes chunks g, g + 4, ... of its output row, and lanes
//     g < planes write one 4-byte value of row tau to plane g (the norm and
//     residual-norm planes), all non-temporal, exactly as the quantiser at
//     d = 128 moves its input rows, packed codes and per-token scalars.  Its
//     time is the floor of a quantise that moves the same bytes this way.
#include <algorithm>

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

__global__ __launch_bounds__(256) void stream_rw_kernel(const u32x4s* __restrict__ src, long rows, int in_chunks,
                                                        u32x4s* __restrict__ dst, int out_chunks,
                                                        float* __restrict__ planes, int nplanes) {
  const int lane = threadIdx.x & 63, tau = lane & 15, g = lane >> 4;
  const long tiles = (rows + 15) >> 4;
  for (long tile = (long)blockIdx.x * 4 + (threadIdx.x >> 6); tile < tiles; tile += (long)gridDim.x * 4) {
    const long r = tile * 16 + tau;
    if (r >= rows) continue;
    const u32x4s* in = src + r * in_chunks;
    u32x4s acc = {0u, 0u, 0u, 0u};
    // Four loads in flight per lane before any is consumed, as in the quantiser.
    for (int c0 = 0; c0 < in_chunks; c0 += 16) {
      u32x4s v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = c0 + 4 * k + g;
        v[k] = c < in_chunks ? __builtin_nontemporal_load(in + c) : u32x4s{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= v[k];
    }
    u32x4s* out = dst + r * out_chunks;
    for (int c = g; c < out_chunks; c += 4) __builtin_nontemporal_store(acc, out + c);
    if (g < nplanes) __builtin_nontemporal_store(__uint_as_float(acc.x & 0x3fffffffu), planes + (long)g * rows + r);
  }
}

}  // namespace

int stream_read_blocks() { return 2048; }

hipError_t launch_stream_rw(const void* src, long rows, int in_row_bytes, void* dst, int out_row_bytes, float* planes,
                            int nplanes, int cus, hipStream_t s) {
  hipLaunchKernelGGL(stream_rw_kernel, dim3(std::max(1, cus * 4)), dim3(256), 0, s,
                     reinterpret_cast<const u32x4s*>(src), rows, in_row_bytes / 16, reinterpret_cast<u32x4s*>(dst),
                     out_row_bytes / 16, planes, nplanes);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(stream_read_blocks()), dim3(256), 0, s,
                     reinterpret_cast<const u32x4s*>(src), bytes / 16, reinterpret_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace tq
