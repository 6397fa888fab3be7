// q4_gemv_skinny: Y[M, N] = X[M, K] . What^T for M <= 8 -- the weight stream
// of autoregressive decode and of speculative verification.
//
// Pages: decode streams every quantized weight once per step and is bound by
// memory bandwidth (page 3, "Qwen3.8-27B at 256K on a 24GB RTX PRO 4000
// SFF", the paragraph on the 432 GB/s ceiling; page 5, section "Why the A8
// artifact matters", on decode processing very few tokens per step), and
// speculative verification scores 1 + d drafted tokens in the same pass
// (page 3, MTP with n_max = 3, i.e. M = 4).
//
// gfx950 design (HBM-bound; VALU only):
//  * A wave is 4 row-slots x 16 lanes.  Lane j of a row-slot owns 32-weight
//    blocks j, j+16, j+32, ... of its rows, so each dwordx4 load of a wave
//    reads 4 rows x 256 contiguous bytes of codes: coalesced 128-bit loads.
//    Every lane carries RL rows, re-using its activation registers RL times.
//  * Activations are staged once per workgroup into LDS in a permuted fp16
//    layout matching the in-register unpack below, plus a per-block bias.
//  * Unpack: (w & 0x000F000F) ^ 0x64086408 flips each nibble's sign bit
//    (two's complement q -> u = q + 8) and inserts the fp16 exponent of 1024
//    (mantissa LSB = 1), giving the pair (1024 + u0, 1024 + u4) in one
//    v_bitop3.  Odd nibbles sit 4 bits higher, so they get the exponent of 64
//    (mantissa LSB = 1/16): (w & 0x00F000F0) ^ 0x54805480 = (64 + u1, 64 + u5).
//    v_dot2_f32_f16 accumulates in fp32 against unscaled fp16 activations and
//    the constant parts (1032 per even, 72 per odd activation) are removed
//    exactly by starting each block's accumulator at -bias.  The
//    block scale multiplies the block partial once (fp32 FMA).
//  * 16-lane DPP rotations reduce each row; K can be split over workgroups
//    (split-K) whose fp32 partials are summed in a fixed order by the last
//    workgroup to arrive (one kernel, deterministic).

#include "q4w_internal.h"
#include <hip/hip_fp16.h>

namespace q4w {
namespace {

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kLanesPerRow = 16;        // lanes sharing one row along K
constexpr int kSlots = 64 / kLanesPerRow;
constexpr int kLdsBudget = 40 * 1024;   // activation staging bytes per workgroup

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Word 3 of a gfx9 buffer resource: 32-bit data format, raw (untyped) access.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // row_ror:1
  return v;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Rows per lane: more rows re-use the activation registers more (less LDS
// traffic per weight) at the cost of fewer workgroups.
template <int M> struct RowsPerLane { static constexpr int value = 4; };

// Occupancy target per M: enough waves per SIMD to keep loads in flight.
template <int M> struct WavesPerEu { static constexpr int value = M <= 2 ? 4 : 3; };

template <int M>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(WavesPerEu<M>::value, 8)))
skinny_kernel(const uint16_t* __restrict__ x, const uint4* __restrict__ codes,
              const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
              float* __restrict__ partial, uint32_t* __restrict__ counters,
              int N, int K, int bps, int S) {
  constexpr int RL = RowsPerLane<M>::value;
  constexpr int kRowsPerWg = kWaves * kSlots * RL;
  extern __shared__ uint4 smem[];

  const int nb = K / kBlock;
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int kb0 = split * bps;
  const int nbs = min(bps, nb - kb0);        // blocks in this slice (>= 1)
  const int steps = (nbs + kLanesPerRow - 1) / kLanesPerRow;
  const int bpad = steps * kLanesPerRow;     // slice length padded to whole steps

  uint4* xs = smem;                                          // [M][4][bpad] fp16 quads
  float* cs = reinterpret_cast<float*>(smem + M * 4 * bpad); // [M][bpad] bias

  // ---- stage the activation slice in the unpack's pair order --------------
  const uint32_t k1032 = 0x64086408u;   // fp16 pair (1032, 1032)
  const uint32_t k72 = 0x54805480u;     // fp16 pair (72, 72)
  for (int u = tid; u < M * bpad; u += kThreads) {
    const int m = u / bpad;
    const int b = u - m * bpad;
    uint4 raw[4];
    if (b < nbs) {
      const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)m * K + (size_t)(kb0 + b) * kBlock);
#pragma unroll
      for (int q = 0; q < 4; ++q) raw[q] = src[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) raw[q] = make_uint4(0, 0, 0, 0);
    }
    float c = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // raw[q] holds elements e0..e7 of code word q as (e1:e0, e3:e2, e5:e4, e7:e6)
      const uint32_t w0 = raw[q].x, w1 = raw[q].y, w2 = raw[q].z, w3 = raw[q].w;
      uint4 o;
      o.x = (w0 & 0xFFFFu) | (w2 << 16);                               // (e0, e4)
      o.y = (w0 >> 16) | (w2 & 0xFFFF0000u);                           // (e1, e5)
      o.z = (w1 & 0xFFFFu) | (w3 << 16);                               // (e2, e6)
      o.w = (w1 >> 16) | (w3 & 0xFFFF0000u);                           // (e3, e7)
      xs[(m * 4 + q) * bpad + b] = o;
      c = dot2(o.x, k1032, c);
      c = dot2(o.y, k72, c);
      c = dot2(o.z, k1032, c);
      c = dot2(o.w, k72, c);
    }
    cs[m * bpad + b] = -c;
  }
  __syncthreads();

  // ---- stream the weights -----------------------------------------------
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int slot = lane >> 4;
  const int j = lane & (kLanesPerRow - 1);
  const int row0 = tile * kRowsPerWg + (wave * kSlots + slot) * RL;

  // Buffer resources cover this workgroup's rows only; a lane whose row is
  // past N reads zeros (hardware range check), so rows need no clamping.
  const int tile_row0 = tile * kRowsPerWg;
  const int rows_here = min(kRowsPerWg, N - tile_row0);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + (size_t)tile_row0 * nb), 0, rows_here * nb * kBlockBytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + (size_t)tile_row0 * nb), 0, rows_here * nb * 2, kRsrcWord3);
  int voff[RL];   // block index (row-local) of this lane's first block, per row
#pragma unroll
  for (int i = 0; i < RL; ++i) voff[i] = (row0 - tile_row0 + i) * nb + kb0 + j;

  float yacc[RL][M];
#pragma unroll
  for (int i = 0; i < RL; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) yacc[i][m] = 0.f;

  // Two register buffers alternate between "in flight" and "being consumed",
  // so the loads of step t+1 overlap the arithmetic of step t without any
  // register copies.  The step offset is wave-uniform (an SGPR).  A lane
  // whose block lies past the slice reads a neighbouring block of the same
  // arrays (or zeros past the end); its LDS activations and bias are zero,
  // so it contributes exactly 0.
  uint4 bufA[RL], bufB[RL];
  uint32_t sA[RL], sB[RL];
  auto load_step = [&](int t, uint4 (&c)[RL], uint32_t (&sc)[RL]) {
#pragma unroll
    for (int i = 0; i < RL; ++i) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rc, voff[i] * kBlockBytes,
                                                          t * kLanesPerRow * kBlockBytes, 0);
      c[i] = make_uint4(v[0], v[1], v[2], v[3]);
      sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff[i] * 2, t * kLanesPerRow * 2, 0);
    }
  };
  auto compute_step = [&](int t, const uint4 (&c)[RL], const uint32_t (&sc)[RL]) {
    const int b = t * kLanesPerRow + j;
    float acc[RL][M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float nc = cs[m * bpad + b];   // holds -bias
#pragma unroll
      for (int i = 0; i < RL; ++i) acc[i][m] = nc;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 xq[M];
#pragma unroll
      for (int m = 0; m < M; ++m) xq[m] = xs[(m * 4 + q) * bpad + b];
#pragma unroll
      for (int i = 0; i < RL; ++i) {
        // (w & mask) ^ (exponent | sign bits): flips each nibble's sign bit
        // (two's complement -> u = q + 8) and inserts an fp16 exponent.
        const uint32_t w = word(c[i], q);
        const uint32_t w8 = w >> 8;
        const uint32_t p0 = (w & 0x000F000Fu) ^ 0x64086408u;   // 1024 + u, nibbles 0, 4
        const uint32_t p1 = (w & 0x00F000F0u) ^ 0x54805480u;   // 64 + u, nibbles 1, 5
        const uint32_t p2 = (w8 & 0x000F000Fu) ^ 0x64086408u;  // 1024 + u, nibbles 2, 6
        const uint32_t p3 = (w8 & 0x00F000F0u) ^ 0x54805480u;  // 64 + u, nibbles 3, 7
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float a = acc[i][m];
          a = dot2(p0, xq[m].x, a);
          a = dot2(p1, xq[m].y, a);
          a = dot2(p2, xq[m].z, a);
          a = dot2(p3, xq[m].w, a);
          acc[i][m] = a;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RL; ++i) {
      const float d = __half2float(__ushort_as_half((unsigned short)sc[i]));
#pragma unroll
      for (int m = 0; m < M; ++m) yacc[i][m] = fmaf(acc[i][m], d, yacc[i][m]);
    }
  };

  // Loads are unconditional (a step past the end reads data it ignores): a
  // conditional load would make the compiler wait for every outstanding load
  // at the merge point and serialize the pipeline.
  load_step(0, bufA, sA);
#pragma unroll 1
  for (int t = 0; t < steps; t += 2) {
    load_step(t + 1, bufB, sB);
    compute_step(t, bufA, sA);
    load_step(t + 2, bufA, sA);
    if (t + 1 < steps) compute_step(t + 1, bufB, sB);
  }

  // ---- reduce the 16 lanes of each row; lane j then stores value j -------
  constexpr int kVals = RL * M;          // (row i, token m) pairs, index i * M + m
  float tot[RL][M];
#pragma unroll
  for (int i = 0; i < RL; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) tot[i][m] = row16_sum(yacc[i][m]);
#pragma unroll
  for (int pass = 0; pass < (kVals + kLanesPerRow - 1) / kLanesPerRow; ++pass) {
    const int idx = pass * kLanesPerRow + j;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < RL; ++i)
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (idx == i * M + m) v = tot[i][m];
    if (idx < kVals) {
      const int i = idx / M;
      const int m = idx - i * M;
      const int n = row0 + i;
      if (n < N) {
        if (S == 1) y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(v));
        else partial[((size_t)split * M + m) * N + n] = v;
      }
    }
  }

  if (S == 1) return;

  // ---- split-K: the last workgroup of this row tile sums the partials ----
  __shared__ int is_last;
  __threadfence();                       // release this thread's partial stores
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&counters[tile], 1u);
    is_last = (prev == (unsigned)(S - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();                       // acquire the other workgroups' partials
  for (int o = tid; o < kRowsPerWg * M; o += kThreads) {
    const int m = o / kRowsPerWg;
    const int n = tile * kRowsPerWg + (o - m * kRowsPerWg);
    if (n < N) {
      float s = 0.f;
      for (int sp2 = 0; sp2 < S; ++sp2)
        s += __hip_atomic_load(&partial[((size_t)sp2 * M + m) * N + n], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(s));
    }
  }
  if (tid == 0) counters[tile] = 0u;    // leave the workspace ready for the next call
}

__global__ void fill_zero_kernel(uint16_t* y, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) y[i] = 0;
}

template <int M>
hipError_t launch_m(const uint16_t* x, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                    int64_t N, int64_t K, const SkinnyPlan& p, void* ws, hipStream_t s) {
  const int bpad = ((p.blocks_per_split + kLanesPerRow - 1) / kLanesPerRow) * kLanesPerRow;
  const size_t lds = (size_t)M * bpad * (4 * sizeof(uint4) + sizeof(float));
  uint32_t* counters = nullptr;
  float* partial = nullptr;
  if (p.splits > 1) {
    counters = reinterpret_cast<uint32_t*>(ws);
    partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.counter_bytes);
  }
  hipLaunchKernelGGL(skinny_kernel<M>, dim3(p.row_tiles, p.splits), dim3(kThreads), lds, s, x,
                     reinterpret_cast<const uint4*>(codes), scales, y, partial, counters, (int)N,
                     (int)K, p.blocks_per_split, p.splits);
  return hipGetLastError();
}

}  // namespace

SkinnyPlan plan_skinny(int M, int64_t N, int64_t K, int split_k) {
  SkinnyPlan p{};
  const int rl = 4;  // RowsPerLane<M>::value for every M
  p.rows_per_wg = kWaves * kSlots * rl;
  p.row_tiles = (int)((N + p.rows_per_wg - 1) / p.rows_per_wg);
  const int nb = (int)(K / kBlock);
  // largest slice whose staged activations fit the LDS budget, in whole steps
  int bps_max = kLdsBudget / (M * (4 * 16 + 4));
  bps_max = (bps_max / kLanesPerRow) * kLanesPerRow;
  int S = split_k > 0 ? split_k : 1;
  if (split_k == 0) {
    const int target_wgs = 512;  // >= 2 workgroups (8 waves) per CU on 256 CUs
    const int want = (target_wgs + p.row_tiles - 1) / p.row_tiles;
    const int cap = nb / kLanesPerRow > 0 ? nb / kLanesPerRow : 1;  // >= one step per slice
    S = want < cap ? want : cap;
    if (S < 1) S = 1;
  }
  int bps = (nb + S - 1) / S;
  if (split_k == 0) bps = ((bps + kLanesPerRow - 1) / kLanesPerRow) * kLanesPerRow;
  if (bps > bps_max) bps = bps_max;
  if (bps < 1) bps = 1;
  p.blocks_per_split = bps;
  p.splits = (nb + bps - 1) / bps;
  if (p.splits > 1) {
    // Counters live in a fixed region at the start of every workspace and
    // partials always start after it, so a workspace shared between shapes
    // never has one shape's partials where another shape's counters are.
    p.counter_bytes = kCounterRegionBytes;
    p.ws_bytes = p.counter_bytes + (size_t)p.splits * M * N * sizeof(float);
  }
  return p;
}

hipError_t launch_skinny(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                         uint16_t* y, int M, int64_t N, int64_t K, const SkinnyPlan& p, void* ws,
                         hipStream_t s) {
  switch (M) {
    case 1: return launch_m<1>(x, codes, scales, y, N, K, p, ws, s);
    case 2: return launch_m<2>(x, codes, scales, y, N, K, p, ws, s);
    case 3: return launch_m<3>(x, codes, scales, y, N, K, p, ws, s);
    case 4: return launch_m<4>(x, codes, scales, y, N, K, p, ws, s);
    case 5: return launch_m<5>(x, codes, scales, y, N, K, p, ws, s);
    case 6: return launch_m<6>(x, codes, scales, y, N, K, p, ws, s);
    case 7: return launch_m<7>(x, codes, scales, y, N, K, p, ws, s);
    case 8: return launch_m<8>(x, codes, scales, y, N, K, p, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill_zero_u16(uint16_t* y, int64_t count, hipStream_t s) {
  const int64_t grid = (count + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)grid), dim3(256), 0, s, y, count);
  return hipGetLastError();
}

}  // namespace q4w
