// A8 prefill route: int8 activations (per token, per 64 channels) against the
// 4-bit block weights on int8 matrix cores, fp32 rescale, fp16 output.
//
// Page 5 ("Qwen3.8-27B on RTX 4090: 5,000 tok/s Prefill Reproduced"),
// section "Why the A8 artifact matters": for large prompt steps activations
// are quantized per token and per 64 channels and fed to an int8
// tensor-core product against the groupwise weights.  Readings (the page
// gives no formulas): sa = fl32(absmax / 127), qa = clamp(round_half_away(
// fl32(x / sa)), -127, 127); weight groups are the same 32-element 4-bit
// blocks; one activation group covers two weight blocks.
//
// gfx950 design:
//  * v_mfma_i32_32x32x32_i8: one instruction = one 32-wide weight block, so
//    every block sum I[m, n, b] comes out exact in int32.
//  * Nibbles become int8 with two bit operations: (w & 0xF0F0F0F0) holds the
//    odd codes times 16 and ((w << 4) & 0xF0F0F0F0) the even codes times 16,
//    both exact signed int8.  The activation tile is stored with the same
//    even/odd permutation inside every 8 channels, so the order of the dot
//    product changes but not its value; the result is 16 * I.
//  * Magic-number descale: the MFMA accumulator input is the constant
//    0x4B400000 (1.5 * 2^23), so the int32 result read as fp32 is exactly
//    12582912 + 16 I; two FMAs per group fold both block scales and remove
//    the offset, one FMA applies the activation scale.
//  * Activations are quantized into the workspace in the MFMA operand order
//    (one 1 KB coalesced load per 32x32 operand); weight codes and scales are
//    staged through LDS with an XOR swizzle (conflict-free 128-bit reads) and
//    halves are exchanged across the wave with v_permlane32_swap.

#include "q4w_internal.h"
#include <hip/hip_fp16.h>

namespace q4w {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float round_half_away(float v) {
  float t = truncf(v);
  if (fabsf(v - t) >= 0.5f) t += copysignf(1.0f, v);
  return t;
}

__device__ __forceinline__ int quant127(float x, float sa) {
  if (sa == 0.0f) return 0;
  float q = round_half_away(x / sa);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return (int)q;
}

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xFFFFu)));
    v[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
  }
}

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
  return a;
}

// ---- row-major quantizer (the exported a8_quantize_act) --------------------
// 8 lanes per (token, 64-channel group); lane e owns channels 8e .. 8e+7.
__global__ void __launch_bounds__(256) act_quant_rowmajor_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t ngroups, int G, int K,
                                                                 int8_t* __restrict__ xq,
                                                                 float* __restrict__ sa) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t grp = t >> 3;
  const int e = threadIdx.x & 7;
  const bool live = grp < ngroups;
  const int64_t m = live ? grp / G : 0;
  const int g = live ? (int)(grp - m * G) : 0;
  const size_t off = (size_t)m * K + (size_t)g * kActGroup + 8 * e;
  float v[8];
  if (live) load8(x + off, v);
  else for (int i = 0; i < 8; ++i) v[i] = 0.f;
  float a = absmax8(v);
  a = fmaxf(a, __shfl_xor(a, 1, 8));
  a = fmaxf(a, __shfl_xor(a, 2, 8));
  a = fmaxf(a, __shfl_xor(a, 4, 8));
  const float s = a / 127.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= ((uint32_t)quant127(v[i], s) & 0xFFu) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= ((uint32_t)quant127(v[4 + i], s) & 0xFFu) << (8 * i);
  if (live) {
    *reinterpret_cast<uint2*>(xq + off) = make_uint2(lo, hi);
    if (e == 0) sa[(size_t)m * G + g] = s;
  }
}

// ---- tiled quantizer (private workspace layout of the GEMM) ----------------
// Layout, for 32-row tile mt, weight block b and MFMA lane l = r + 32 h:
//   xq_t[((mt * nb + b) * 64 + l) * 16 + s] = qa[32 mt + r][32 b + 16 h + perm(s)]
//   perm = 0,2,4,6,1,3,5,7, 8,10,12,14,9,11,13,15  (matches the nibble unpack)
//   sa_t[(mt * G + g) * 32 + r] = sa[32 mt + r][g]
// Rows at or beyond M are written as zeros.  One wave per (mt, g): lane
// (r, h) quantizes channels 16h..16h+15 of both blocks of group g for row r;
// the group absmax pairs lane r with lane r + 32.
__global__ void __launch_bounds__(64) act_quant_tiled_kernel(const uint16_t* __restrict__ x, int M,
                                                             int K, uint4* __restrict__ xq_t,
                                                             float* __restrict__ sa_t) {
  const int G = K / kActGroup;
  const int nb = K / kBlock;
  const int mt = blockIdx.y;
  const int g = blockIdx.x;
  const int l = threadIdx.x;
  const int r = l & 31;
  const int h = l >> 5;
  const int m = mt * kA8TileM + r;
  float v[2][16];
  if (m < M) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const uint16_t* p = x + (size_t)m * K + (size_t)g * kActGroup + bi * kBlock + 16 * h;
      float t0[8], t1[8];
      load8(p, t0);
      load8(p + 8, t1);
#pragma unroll
      for (int i = 0; i < 8; ++i) { v[bi][i] = t0[i]; v[bi][8 + i] = t1[i]; }
    }
  } else {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[bi][i] = 0.f;
  }
  float a = 0.f;
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(v[bi][i]));
  a = fmaxf(a, __shfl_xor(a, 32, 64));
  const float s = a / 127.0f;
  constexpr int perm[16] = {0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15};
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    uint32_t wv[4] = {0, 0, 0, 0};
#pragma unroll
    for (int sidx = 0; sidx < 16; ++sidx)
      wv[sidx >> 2] |= ((uint32_t)quant127(v[bi][perm[sidx]], s) & 0xFFu) << (8 * (sidx & 3));
    const int b = 2 * g + bi;
    xq_t[((size_t)mt * nb + b) * 64 + l] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  if (h == 0) sa_t[((size_t)mt * G + g) * 32 + r] = s;
}

// ---- int8 MFMA GEMM --------------------------------------------------------
constexpr int kTM = 128;          // workgroup tile rows (tokens)
constexpr int kTN = 128;          // workgroup tile columns (output features)
constexpr int kChunkBlocks = 8;   // weight blocks staged per LDS chunk (256 K)
constexpr float kMagic = 12582912.0f;   // 0x4B400000 = 1.5 * 2^23

__device__ __forceinline__ uint32_t lo_codes(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t hi_codes(uint32_t w) { return w & 0xF0F0F0F0u; }

template <bool kDebug>
__global__ void __launch_bounds__(256)
a8w4_gemm_kernel(const uint4* __restrict__ xq_t, const float* __restrict__ sa_t,
                 const uint4* __restrict__ codes, const uint16_t* __restrict__ scales,
                 uint16_t* __restrict__ y, int32_t* __restrict__ acc_dbg, int M, int N, int K,
                 int mtiles, int ntiles) {
  __shared__ uint4 lds_b[kTN * kChunkBlocks];        // codes, 16 B per (row, block), swizzled
  __shared__ uint4 lds_s[kTN];                       // 8 fp16 scales per row

  const int nb = K / kBlock;
  const int G = K / kActGroup;
  const int tid = threadIdx.x;

  // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
  // give each XCD a contiguous range of tiles (column-major: one weight tile
  // is re-used across all token tiles inside one XCD's L2).
  const int total = mtiles * ntiles;
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int mt = bid % mtiles;
  const int nt = bid / mtiles;

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1;          // 2 x 2 waves, each 64 x 64
  const int wn = wave & 1;
  const int j = lane & 31;
  const int h = lane >> 5;
  const int n_base = nt * kTN;
  const int mtile32[2] = {(mt * kTM + wm * 64) / kA8TileM, (mt * kTM + wm * 64) / kA8TileM + 1};

  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = 0x4B400000;

  float acc[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  for (int kc = 0; kc < nb; kc += kChunkBlocks) {
    const int nblk = min(kChunkBlocks, nb - kc);
    __syncthreads();
    // cooperative stage of codes: kTN rows x 8 blocks, unit u of row r at u ^ (r & 7)
#pragma unroll
    for (int it = 0; it < (kTN * kChunkBlocks) / 256; ++it) {
      const int idx = it * 256 + tid;
      const int row = idx >> 3;
      const int u = idx & 7;
      const int n = min(n_base + row, N - 1);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (u < nblk) v = codes[(size_t)n * nb + kc + u];
      lds_b[row * kChunkBlocks + (u ^ (row & 7))] = v;
    }
    if (!kDebug && tid < kTN) {
      const int n = min(n_base + tid, N - 1);
      uint32_t sv[4] = {0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < kChunkBlocks; ++u)
        if (u < nblk) sv[u >> 1] |= (uint32_t)scales[(size_t)n * nb + kc + u] << (16 * (u & 1));
      lds_s[tid] = make_uint4(sv[0], sv[1], sv[2], sv[3]);
    }
    __syncthreads();

    for (int g2 = 0; g2 < nblk; g2 += 2) {
      const int b0 = kc + g2;
      const int g = b0 >> 1;
      // activation operands (two 32-row tiles x two blocks) and scales
      v4i av[2][2];
      float sav[2][16];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
          const uint4 t = xq_t[((size_t)mtile32[mi] * nb + b0 + bi) * 64 + lane];
          av[mi][bi] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
        }
        const float4* sp = reinterpret_cast<const float4*>(sa_t + ((size_t)mtile32[mi] * G + g) * 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 f = sp[2 * r + h];
          sav[mi][4 * r + 0] = f.x; sav[mi][4 * r + 1] = f.y;
          sav[mi][4 * r + 2] = f.z; sav[mi][4 * r + 3] = f.w;
        }
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = wn * 64 + ni * 32 + j;
        // lane (j, h) reads the whole 16 B of block b0 + h, then the two halves
        // of the wave swap so lane (j, h) holds K-half h of block b0 and of b0+1
        const uint4 raw = lds_b[row * kChunkBlocks + ((g2 + h) ^ (row & 7))];
        const auto s02 = __builtin_amdgcn_permlane32_swap(raw.x, raw.z, false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(raw.y, raw.w, false, false);
        const uint32_t p0 = s02[0], p1 = s13[0];   // block b0, half h
        const uint32_t q0 = s02[1], q1 = s13[1];   // block b0 + 1, half h
        const v4i bv0 = v4i{(int)lo_codes(p0), (int)hi_codes(p0), (int)lo_codes(p1), (int)hi_codes(p1)};
        const v4i bv1 = v4i{(int)lo_codes(q0), (int)hi_codes(q0), (int)lo_codes(q1), (int)hi_codes(q1)};
        const uint4 sc = lds_s[row];
        const uint32_t sw = (g2 >> 1) == 0 ? sc.x : (g2 >> 1) == 1 ? sc.y : (g2 >> 1) == 2 ? sc.z : sc.w;
        // the B operand carries 16 * q, fold the 1/16 into the scales (exact)
        const float d0 = __half2float(__ushort_as_half((unsigned short)(sw & 0xFFFFu))) * 0.0625f;
        const float d1 = __half2float(__ushort_as_half((unsigned short)(sw >> 16))) * 0.0625f;
        const float nc = -kMagic * (d0 + d1);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const v16i D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mi][0], bv0, magic, 0, 0, 0);
          const v16i D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mi][1], bv1, magic, 0, 0, 0);
          if (kDebug) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int mrow = mtile32[mi] * kA8TileM + 8 * (v >> 2) + 4 * h + (v & 3);
              const int ncol = n_base + wn * 64 + ni * 32 + j;
              if (mrow < M && ncol < N) {
                int32_t* o = acc_dbg + ((size_t)mrow * N + ncol) * nb + b0;
                o[0] = (D0[v] - 0x4B400000) >> 4;
                o[1] = (D1[v] - 0x4B400000) >> 4;
              }
            }
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float s = fmaf(__int_as_float(D0[v]), d0, fmaf(__int_as_float(D1[v]), d1, nc));
              acc[mi][ni][v] = fmaf(s, sav[mi][v], acc[mi][ni][v]);
            }
          }
        }
      }
    }
  }

  if (kDebug) return;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int ncol = n_base + wn * 64 + ni * 32 + j;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int mrow = mtile32[mi] * kA8TileM + 8 * (v >> 2) + 4 * h + (v & 3);
        if (mrow < M && ncol < N)
          y[(size_t)mrow * N + ncol] = __half_as_ushort(__float2half_rn(acc[mi][ni][v]));
      }
    }
}

}  // namespace

int64_t a8_padded_rows(int64_t M) { return ((M + kTM - 1) / kTM) * kTM; }

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t a8_ws_bytes(int64_t M, int64_t K) {
  const int64_t mp = a8_padded_rows(M);
  return align256((size_t)mp * K) + align256((size_t)mp * (K / kActGroup) * sizeof(float));
}

hipError_t launch_act_quant_rowmajor(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* sa,
                                     hipStream_t s) {
  const int G = (int)(K / kActGroup);
  const int64_t ngroups = M * G;
  const int64_t grid = (ngroups * 8 + 255) / 256;
  hipLaunchKernelGGL(act_quant_rowmajor_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, ngroups, G,
                     (int)K, xq, sa);
  return hipGetLastError();
}

hipError_t launch_act_quant_tiled(const uint16_t* x, int64_t M, int64_t K, void* ws, hipStream_t s) {
  const int64_t mp = a8_padded_rows(M);
  uint4* xq_t = reinterpret_cast<uint4*>(ws);
  float* sa_t = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)mp * K));
  hipLaunchKernelGGL(act_quant_tiled_kernel, dim3((unsigned)(K / kActGroup), (unsigned)(mp / kA8TileM)),
                     dim3(64), 0, s, x, (int)M, (int)K, xq_t, sa_t);
  return hipGetLastError();
}

hipError_t launch_a8w4_gemm(const void* ws, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                            int32_t* acc_debug, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  const int64_t mp = a8_padded_rows(M);
  const uint4* xq_t = reinterpret_cast<const uint4*>(ws);
  const float* sa_t = reinterpret_cast<const float*>(static_cast<const char*>(ws) + align256((size_t)mp * K));
  const int mtiles = (int)(mp / kTM);
  const int ntiles = (int)((N + kTN - 1) / kTN);
  const dim3 grid((unsigned)(mtiles * ntiles));
  if (acc_debug)
    hipLaunchKernelGGL(a8w4_gemm_kernel<true>, grid, dim3(256), 0, s, xq_t, sa_t,
                       reinterpret_cast<const uint4*>(codes), scales, y, acc_debug, (int)M, (int)N,
                       (int)K, mtiles, ntiles);
  else
    hipLaunchKernelGGL(a8w4_gemm_kernel<false>, grid, dim3(256), 0, s, xq_t, sa_t,
                       reinterpret_cast<const uint4*>(codes), scales, y, acc_debug, (int)M, (int)N,
                       (int)K, mtiles, ntiles);
  return hipGetLastError();
}

}  // namespace q4w
