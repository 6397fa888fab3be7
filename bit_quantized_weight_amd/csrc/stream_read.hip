// q4w_stream_read: a plain streaming read of a device buffer, the measured
// ceiling that the HBM-bound kernels of this library are compared with.  It
// is a measurement helper, not a step of the method.
//
// Every thread keeps four 16-byte loads in flight, grid-stride over the
// buffer, so at any time the whole chip reads one narrow window of it; each
// workgroup writes the XOR of the 32-bit words it read (a checksum, which
// also keeps the loads from being optimized away).

#include "q4w_internal.h"

namespace q4w {
namespace {

constexpr int kReadUnroll = 4;

__global__ void stream_read_kernel(const uint4* __restrict__ p, size_t n16, uint32_t* __restrict__ out) {
  __shared__ uint32_t part[16];
  const size_t nthreads = (size_t)gridDim.x * blockDim.x;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t x = 0;
  for (size_t base = tid; base < n16; base += nthreads * kReadUnroll) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const size_t i = base + (size_t)u * nthreads;
      v[u] = i < n16 ? p[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // XOR over the wave, then over the workgroup's waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int grid, int block,
                              hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3((unsigned)block), 0, s,
                     static_cast<const uint4*>(buf), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace q4w
