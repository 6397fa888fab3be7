// q4w_stream_read: a plain streaming read of a device buffer, the measured
// ceiling that the HBM-bound kernels of this library are compared with.  It
// is a measurement helper, not a step of the method.
//
// Every thread keeps four 16-byte loads in flight, grid-stride over the
// buffer, so at any time the whole chip reads one narrow window of it; each
// wave writes the XOR of the 32-bit words it read (a checksum, which also
// keeps the loads from being optimized away), reduced in registers so that
// the launch ends without LDS round trips or a barrier.

#include "q4w_internal.h"

namespace q4w {
namespace {

constexpr int kReadUnroll = 4;

__global__ void stream_read_kernel(const uint4* __restrict__ p, size_t n16, uint32_t* __restrict__ out) {
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
  // XOR over the wave in registers (no LDS round trips, no barrier): rotations
  // within each row of 16 lanes, then across rows (lanes l ^ 16, l ^ 32).
  x ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);   // row_ror:8
  x ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false);   // row_ror:4
  x ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x122, 0xF, 0xF, false);   // row_ror:2
  x ^= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x121, 0xF, 0xF, false);   // row_ror:1
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = r16[0] ^ r16[1];
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = r32[0] ^ r32[1];
  if ((threadIdx.x & 63) == 0) out[(size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = x;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int grid, int block,
                              hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3((unsigned)block), 0, s,
                     static_cast<const uint4*>(buf), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace q4w
