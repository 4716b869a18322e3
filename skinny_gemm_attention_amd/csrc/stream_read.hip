// Streaming-read reference kernel: the bandwidth a plain read of HBM reaches
// on this device, the yardstick for the achieved bandwidth of the kernels of
// the path (it computes nothing of the method).
//
// 65536 workgroups of 512 threads walk the buffer in a grid-stride loop, one
// 16-byte non-temporal load per thread and step, so the device reads one
// contiguous window that moves through the buffer (measured on MI355X over
// 2 GB: 7.0 TB/s; 2048 workgroups of 256 threads with four loads per step
// reached 6.0 TB/s, larger grids and one load per thread read fastest). The
// XOR of the words a workgroup read is stored to its sink word, which keeps
// every load live.
#include "launch.hpp"

namespace attnres {

constexpr int kStreamThreads = 512;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                     size_t n16, unsigned* sink) {
  __shared__ unsigned part[kStreamThreads / 64];
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n16; i += stride)
    acc ^= __builtin_nontemporal_load(src + i);
  unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) t ^= part[w];
    sink[blockIdx.x] = t;
  }
}

hipError_t launch_stream_read(const void* src, size_t bytes, unsigned* sink, int grid,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace attnres
