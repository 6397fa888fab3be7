// q4_pack: fp32 weights -> 4-bit codes + fp16 block scales.
//
// The 4-bit block format of the decode weight stream (the pages name the
// Q4_0 family -- page 3, "Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF",
// the paragraph on public GGUFs -- without defining it).  Per 32-weight block
// along K: d = fp16_RNE(fl32(absmax / 7)), q = clamp(round_half_away(
// fl32(w / d)), -8, 7), all zero when d == 0; code 2j in the low nibble of
// byte j, code 2j+1 in the high nibble.
//
// One-time preparation, not on the timed path.  Layout: 8 lanes per block,
// each lane owns 4 consecutive weights (one float4), so a wave reads 2 KB of
// contiguous fp32 per instruction and writes 128 contiguous code bytes.
// Bit-exactness relies on IEEE division (no fast-math) and RNE fp16 rounding.

#include "q4w_internal.h"
#include <hip/hip_fp16.h>

namespace q4w {
namespace {

__device__ __forceinline__ float round_half_away(float v) {
  float t = truncf(v);
  // v - t is exact for every fp32 v (|v| < 2^23 or v already integral).
  if (fabsf(v - t) >= 0.5f) t += copysignf(1.0f, v);
  return t;
}

__global__ void __launch_bounds__(256) pack_kernel(const float4* __restrict__ w, int64_t nblocks_total,
                                                   uint32_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scales) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = tid >> 3;          // global block index (row-major over [N, K/32])
  const int part = threadIdx.x & 7;      // which 4 weights of the block
  const bool live = blk < nblocks_total;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live) v = w[blk * 8 + part];
  float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  // absmax over the 8 lanes of the block (lane groups of 8 are aligned)
  a = fmaxf(a, __shfl_xor(a, 1, 8));
  a = fmaxf(a, __shfl_xor(a, 2, 8));
  a = fmaxf(a, __shfl_xor(a, 4, 8));
  const __half dh = __float2half_rn(a / 7.0f);
  const float d = __half2float(dh);
  uint32_t nib = 0;
  if (d != 0.0f) {
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float q = round_half_away(e[i] / d);
      q = fminf(fmaxf(q, -8.0f), 7.0f);
      nib |= ((uint32_t)((int)q) & 0xFu) << (4 * i);
    }
  }
  // lane part holds 4 nibbles = 2 bytes; lanes 2p and 2p+1 form code word p.
  const uint32_t other = __shfl_xor(nib, 1, 8);
  if (live && (part & 1) == 0) codes[blk * 4 + (part >> 1)] = nib | (other << 16);
  if (live && part == 0) scales[blk] = __half_as_ushort(dh);
}

}  // namespace

hipError_t launch_pack(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales,
                       hipStream_t s) {
  const int64_t nblocks = N * (K / kBlock);
  // Blocks are independent, so a large matrix is packed in pieces of at most
  // 2^26 blocks: a launch's work-item count (8 per block) stays below 2^32.
  constexpr int64_t kPiece = int64_t(1) << 26;
  for (int64_t b0 = 0; b0 < nblocks; b0 += kPiece) {
    const int64_t nb = nblocks - b0 < kPiece ? nblocks - b0 : kPiece;
    const int64_t grid = (nb * 8 + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(w + b0 * kBlock), nb,
                       reinterpret_cast<uint32_t*>(codes + b0 * (kBlock / 2)), scales + b0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace q4w
