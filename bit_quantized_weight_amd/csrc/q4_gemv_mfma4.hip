// q4_gemv_skinny at M = 4..7 (and M = 3 rows that need splitting) on
// 4 x 4 x 4 matrix-core blocks.
//
// Same operation and pages as q4_gemv.hip: decode and speculative verify
// stream every quantized weight once per step (page 3, "Qwen3.8-27B at 256K
// on a 24GB RTX PRO 4000 SFF", the paragraph on the 432 GB/s ceiling, and MTP
// with n_max = 3, i.e. M = 4).
//
// gfx950 design:
//  * v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4 x 4 x 4 products.  Block
//    b of the instruction is lanes 4b..4b+3; lane 4b + i supplies row i of A
//    and column i of B and receives column i of D (rows 0..3).  Here A is the
//    (up to 4) activation rows and B four weight rows, so no operand row is
//    padding at M = 4, and the v_dot2 form's M dot products per weight
//    pair become one matrix instruction per 4 x 4 x 4 product.  M = 5..7
//    take a second A operand (rows 4..7) against the same unpacked B.
//  * Lane 4b + i of a wave owns weight rows 8w + i and 8w + 4 + i of its
//    workgroup tile (two 4-row groups that share the A operand) and 32-weight
//    block b of every 16-block step, so one 128-bit load of a wave reads 4
//    rows x 256 contiguous bytes of codes.  All of a slice's steps
//    are requested up front; lanes past the end of the slice use an
//    out-of-range buffer offset (zeros, no memory request).
//  * Unpack as in the v_dot2 kernel: one v_bitop3 per fp16 pair gives
//    (1024 + q + 8) for even and (64 + q + 8) for odd nibbles; a block's 8
//    products accumulate on top of -bias (the constant parts times the
//    activations), then the block scale multiplies the block sum (fp32 FMA).
//  * Activations are staged once per workgroup into LDS in the unpack's pair
//    order, with the per-block bias; their loads go out before the weights'.
//  * Lanes of the same weight row are summed by DPP and swizzle in a fixed
//    order; split-K partials are summed in slice order by the last workgroup
//    to arrive (csrc/splitk.h).

#include "q4w_internal.h"
#include "splitk.h"
#include <hip/hip_fp16.h>

namespace q4w {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStepBlocks = 16;            // 32-weight blocks per step (one per lane group)
constexpr int kFixupBatch = 16;
constexpr int kMaxSliceSteps = 10;         // the deepest copy of the kernel
static_assert(kMaxSliceSteps * kStepBlocks == kMfma4SliceBlocks, "one-slice rows");
constexpr int kSplitSliceSteps = 4;        // longest slice of a split row
// Deepest copy with two row groups: with two A operands (M > 4) the 8- and
// 10-step copies would spill registers.
__host__ __device__ constexpr int max_pair_steps(int M) { return M > 4 ? 6 : kMaxSliceSteps; }
// Activation entries per block in LDS, and the slot of row m in block b.
// Up to M = 4 the rows sit in order (a stride of M entries per block).  With
// two A operands (M = 5..7) a stride of M would make the 64 lanes of an
// operand read (lane 4 blk + c reads row c of block blk) collide on banks,
// so each block takes 8 entries and row m sits at slot (m + 4 (b0 ^ b1)) % 8,
// b0 and b1 the low bits of b: every operand read then touches distinct
// banks (checked for 32 and 64 banks).
__host__ __device__ constexpr int row_stride(int M) { return M > 4 ? 8 : M; }
__host__ __device__ constexpr int row_slot(int M, int m, int b) {
  return M > 4 ? (m + 4 * ((b ^ (b >> 1)) & 1)) & 7 : m;
}
constexpr int kWideTileMinWgs = 512;       // 64-row tiles only with this many workgroups
constexpr int kMinWgs = 256;               // one workgroup per CU
constexpr int kCachePolicyNT = 2;          // non-temporal: codes are read once, in whole lines
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

__device__ __forceinline__ h4 halves(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(h4, v2u{lo, hi});
}

// Sum over the 16 lanes of a wave that hold the same weight row (lane & 3):
// within each DPP row of 16 lanes, then across the four rows.
__device__ __forceinline__ float row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // lane ^ 16
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Slices of at most P steps: every load of a slice is in flight at once.
// kRowGroups: 4-row groups per wave, which share the A operand.
template <int M, int P, int kRowGroups>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(P > 8 ? 3 : 4, 8)))
mfma4_skinny_kernel(const uint16_t* __restrict__ x, const uint4* __restrict__ codes,
                    const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
                    float* __restrict__ partial, uint32_t* __restrict__ counters, int N, int K,
                    int bps, int S) {
  static_assert(M >= 1 && M <= 8, "one or two 4-row A operands");
  constexpr int kASets = (M + 3) / 4;        // A operands: activation rows 4j..4j+3
  constexpr int MP = 4 * kASets;             // bias entries per block
  constexpr int kRowsPerWg = 4 * kRowGroups * kWaves;
  extern __shared__ uint4 smem[];

  const int nb = K / kBlock;
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int kb0 = split * bps;
  const int nbs = min(bps, nb - kb0);        // blocks in this slice (>= 1)
  const int steps = (nbs + kStepBlocks - 1) / kStepBlocks;
  const int bpad = steps * kStepBlocks;

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 3;                    // weight row within the wave, and A row
  const int blk = lane >> 2;                 // block within a step
  const int tile_row0 = tile * kRowsPerWg;
  const int row0 = wave * 4 * kRowGroups + c;   // tile-local weight row of group 0 (+ 4 r)

  const int rows_here = min(kRowsPerWg, N - tile_row0);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + (size_t)tile_row0 * nb), 0, rows_here * nb * kBlockBytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + (size_t)tile_row0 * nb), 0, rows_here * nb * 2, kRsrcWord3);
  uint32_t vblk[kRowGroups];                 // this lane's block in step 0, per row group
#pragma unroll
  for (int r = 0; r < kRowGroups; ++r) vblk[r] = (uint32_t)((row0 + 4 * r) * nb + kb0 + blk);

  // ---- activation loads first: items (row m, block b) of this slice -------
  constexpr int kItems = (M * P * kStepBlocks + kThreads - 1) / kThreads;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, M * K * 2, kRsrcWord3);
  uint4 raw[kItems][4];
  // (A block of its own: the compiler keeps these loads ahead of the weight
  // loads only when they cannot be scheduled together; nbs >= 1 always.)
  if (nbs > 0) {
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int u = tid + it * kThreads;
      const int b = u / M;
      const int m = u - b * M;
      const bool valid = u < M * bpad && b < nbs;
      const uint32_t xo = valid ? (uint32_t)(m * K + (kb0 + b) * kBlock) * 2 : kOutOfRange;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, q * 16, 0);
        raw[it][q] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  } else {
#pragma unroll
    for (int it = 0; it < kItems; ++it)
#pragma unroll
      for (int q = 0; q < 4; ++q) raw[it][q] = make_uint4(0, 0, 0, 0);
  }

  // ---- weight loads: every step of the slice ------------------------------
  uint4 cw[P][kRowGroups];
  uint32_t sw[P][kRowGroups];
#pragma unroll
  for (int t = 0; t < P; ++t) {
    const bool live = t * kStepBlocks + blk < nbs;
#pragma unroll
    for (int r = 0; r < kRowGroups; ++r) {
      const uint32_t vo = live ? vblk[r] * kBlockBytes : kOutOfRange;
      const uint32_t so = live ? vblk[r] * 2 : kOutOfRange;
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, t * kStepBlocks * kBlockBytes, kCachePolicyNT);
      cw[t][r] = make_uint4(v[0], v[1], v[2], v[3]);
      sw[t][r] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, t * kStepBlocks * 2, 0);
    }
  }

  // ---- stage: xs[q][b][m] (16 bytes each), bias[b][MP] -----------------------
  // (m fastest, then b: the 64 lanes of an operand read, lane 4 blk + c, touch
  // one contiguous run of 16-byte entries, so the LDS reads are conflict-free)
  uint4* xs = smem;
  constexpr int MS = row_stride(M);
  float* bias = reinterpret_cast<float*>(smem + bpad * MS * 4);
  const uint32_t k1032 = 0x64086408u;   // fp16 pair (1032, 1032)
  const uint32_t k72 = 0x54805480u;     // fp16 pair (72, 72)
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int u = tid + it * kThreads;
    if (u < M * bpad) {
      const int b = u / M;
      const int m = u - b * M;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // raw holds elements e0..e7 of code word q as (e1:e0, e3:e2, e5:e4, e7:e6)
        const uint32_t w0 = raw[it][q].x, w1 = raw[it][q].y, w2 = raw[it][q].z, w3 = raw[it][q].w;
        uint4 o;
        o.x = (w0 & 0xFFFFu) | (w2 << 16);       // (e0, e4)
        o.y = (w0 >> 16) | (w2 & 0xFFFF0000u);   // (e1, e5)
        o.z = (w1 & 0xFFFFu) | (w3 << 16);       // (e2, e6)
        o.w = (w1 >> 16) | (w3 & 0xFFFF0000u);   // (e3, e7)
        xs[(q * bpad + b) * MS + row_slot(M, m, b)] = o;
        s = dot2(o.x, k1032, s);
        s = dot2(o.y, k72, s);
        s = dot2(o.z, k1032, s);
        s = dot2(o.w, k72, s);
      }
      bias[b * MP + m] = -s;
    }
  }
  __syncthreads();

  // A rows past M read row 4 j, the set's first (their products land in D
  // rows that are dropped); a step adds 16 blocks, which keeps b0 and b1.
  const uint4* xa[kASets];                           // + word q: q * bpad * MS; + step t: t * kStepBlocks * MS
#pragma unroll
  for (int j = 0; j < kASets; ++j) xa[j] = xs + blk * MS + row_slot(M, 4 * j + c < M ? 4 * j + c : 4 * j, blk);
  const float* ba = bias + blk * MP;                 // + step t: t * kStepBlocks * MP

  float yacc[kRowGroups][M];
#pragma unroll
  for (int r = 0; r < kRowGroups; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) yacc[r][m] = 0.f;
#pragma unroll
  for (int t = 0; t < P; ++t) {
    if (t < steps) {
      const float* bt = ba + t * kStepBlocks * MP;
      f4 d[kRowGroups][kASets];
#pragma unroll
      for (int j = 0; j < kASets; ++j) {
        const f4 nb4 = f4{bt[4 * j], bt[4 * j + 1], bt[4 * j + 2], bt[4 * j + 3]};   // -bias, rows 4j..4j+3
#pragma unroll
        for (int r = 0; r < kRowGroups; ++r) d[r][j] = nb4;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 a[kASets];
#pragma unroll
        for (int j = 0; j < kASets; ++j) a[j] = xa[j][t * kStepBlocks * MS + q * bpad * MS];
#pragma unroll
        for (int r = 0; r < kRowGroups; ++r) {
          const uint32_t w = word(cw[t][r], q);
          const uint32_t w8 = w >> 8;
          const uint32_t p0 = (w & 0x000F000Fu) ^ 0x64086408u;   // 1024 + u, nibbles 0, 4
          const uint32_t p1 = (w & 0x00F000F0u) ^ 0x54805480u;   // 64 + u, nibbles 1, 5
          const uint32_t p2 = (w8 & 0x000F000Fu) ^ 0x64086408u;  // nibbles 2, 6
          const uint32_t p3 = (w8 & 0x00F000F0u) ^ 0x54805480u;  // nibbles 3, 7
#pragma unroll
          for (int j = 0; j < kASets; ++j) {
            d[r][j] = __builtin_amdgcn_mfma_f32_4x4x4f16(halves(a[j].x, a[j].y), halves(p0, p1), d[r][j], 0, 0, 0);
            d[r][j] = __builtin_amdgcn_mfma_f32_4x4x4f16(halves(a[j].z, a[j].w), halves(p2, p3), d[r][j], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kRowGroups; ++r) {
        const float s = __half2float(__ushort_as_half((unsigned short)sw[t][r]));
#pragma unroll
        for (int m = 0; m < M; ++m) yacc[r][m] = fmaf(d[r][m / 4][m % 4], s, yacc[r][m]);
      }
    }
  }

  // ---- sum the 16 lanes of each row; lane (blk = r M + m, c) stores ------
  constexpr int kVals = kRowGroups * M;
  static_assert(kVals <= kStepBlocks, "one store pass");
  float v = 0.f;
#pragma unroll
  for (int r = 0; r < kRowGroups; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float sum = row_sum(yacc[r][m]);
      if (blk == r * M + m) v = sum;
    }
  if (blk < kVals) {
    const int r = blk / M;
    const int m = blk - r * M;
    const int n = tile_row0 + row0 + 4 * r;
    if (n < N) {
      if (S == 1) y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(v));
      else
        __hip_atomic_store(&partial[((size_t)split * M + m) * N + n], v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (S == 1) return;

  // ---- split-K: the last workgroup of this row tile sums the partials ----
  __shared__ int is_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == (unsigned)(S - 1));
  }
  __syncthreads();
  if (!is_last) return;
  fixup_tile<kRowsPerWg, M, kThreads, kFixupBatch>(partial, y, N, S, tile_row0);
  if (tid == 0)
    __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int M, int P, int R>
hipError_t launch_p(const uint16_t* x, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                    int64_t N, int64_t K, const SkinnyPlan& p, void* ws, hipStream_t s) {
  const int bpad = ((p.blocks_per_split + kStepBlocks - 1) / kStepBlocks) * kStepBlocks;
  const size_t lds = (size_t)bpad * (row_stride(M) * 4 * sizeof(uint4) + 4 * ((M + 3) / 4) * sizeof(float));
  uint32_t* counters = nullptr;
  float* partial = nullptr;
  if (p.splits > 1) {
    counters = reinterpret_cast<uint32_t*>(ws);
    partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.counter_bytes);
  }
  hipLaunchKernelGGL((mfma4_skinny_kernel<M, P, R>), dim3(p.row_tiles, p.splits), dim3(kThreads), lds, s,
                     x, reinterpret_cast<const uint4*>(codes), scales, y, partial, counters, (int)N,
                     (int)K, p.blocks_per_split, p.splits);
  return hipGetLastError();
}

template <int M, int R>
hipError_t launch_mr(const uint16_t* x, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                     int64_t N, int64_t K, const SkinnyPlan& p, void* ws, hipStream_t s) {
  const int steps = (p.blocks_per_split + kStepBlocks - 1) / kStepBlocks;
  if (steps <= 4) return launch_p<M, 4, R>(x, codes, scales, y, N, K, p, ws, s);
  if (steps <= 6) return launch_p<M, 6, R>(x, codes, scales, y, N, K, p, ws, s);
  if constexpr (R == 1 || max_pair_steps(M) >= kMaxSliceSteps) {
    if (steps <= 8) return launch_p<M, 8, R>(x, codes, scales, y, N, K, p, ws, s);
    if (steps <= kMaxSliceSteps) return launch_p<M, kMaxSliceSteps, R>(x, codes, scales, y, N, K, p, ws, s);
  }
  return hipErrorInvalidValue;
}

template <int M>
hipError_t launch_m(const uint16_t* x, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                    int64_t N, int64_t K, const SkinnyPlan& p, void* ws, hipStream_t s) {
  if (p.rows_per_wg == 16 * kWaves) {   // four row groups: built for short slices and M <= 4 only
    if constexpr (M <= 4) {
      if ((p.blocks_per_split + kStepBlocks - 1) / kStepBlocks <= kSplitSliceSteps)
        return launch_p<M, kSplitSliceSteps, 4>(x, codes, scales, y, N, K, p, ws, s);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (M == 3) {
    // M = 3 comes here only for rows split by the default plan (a forced
    // split_k keeps M = 3 on the v_dot2 kernel): slices of at most 4 steps on
    // two or four row groups, so no other copy is built.
    if (p.rows_per_wg == 8 * kWaves &&
        (p.blocks_per_split + kStepBlocks - 1) / kStepBlocks <= kSplitSliceSteps)
      return launch_p<M, kSplitSliceSteps, 2>(x, codes, scales, y, N, K, p, ws, s);
    return hipErrorInvalidValue;
  } else {
    if (p.rows_per_wg == 8 * kWaves) return launch_mr<M, 2>(x, codes, scales, y, N, K, p, ws, s);
    return launch_mr<M, 1>(x, codes, scales, y, N, K, p, ws, s);
  }
}

}  // namespace

// Split plan: one slice when a row fits the deepest copy (10 steps of 16
// blocks), else slices of at most 4 steps, on 64-row tiles when that still
// gives kWideTileMinWgs workgroups and on 32-row tiles otherwise; more slices
// only below kMinWgs workgroups.  split_k > 0 asks for that many slices
// (raised when a slice would be longer than the deepest copy) on 32-row tiles.
SkinnyPlan plan_skinny_mfma4(int M, int64_t N, int64_t K, int split_k) {
  SkinnyPlan p{};
  p.route = kRouteMfma4;
  const int nb = (int)(K / kBlock);
  const int steps_total = (nb + kStepBlocks - 1) / kStepBlocks;
  // One 4-row group per wave (16-row tiles) on one-slice rows; when K is
  // split, four groups (64-row tiles) if there are enough workgroups, else
  // two.  Measured at M = 4, K = 17408 (us): N = 5120 17.39 with slices of 8
  // steps on 32-row tiles, 15.31 with slices of 4, 15.16 with slices of 4 on
  // 64-row tiles (720 workgroups); N = 8192 21.91, 21.37, 20.24; N = 2560
  // (360 workgroups on 64-row tiles) 11.23, 10.00, 10.88.  The one-slice
  // shapes (K = 5120) measured no better split at M = 4.  With two A
  // operands (M = 5..7) rows of more than 4 steps are split too (M = 5,
  // K = 5120, us: N = 17408 20.95 -> 17.15, N = 7168 10.49 -> 9.98).
  const int one_slice_steps = M > 4 ? kSplitSliceSteps : kMaxSliceSteps;
  const bool split = split_k > 1 || (split_k <= 0 && steps_total > one_slice_steps);
  int S = 1;
  int groups = split ? 2 : 1;
  if (split_k > 0) {
    S = split_k;
  } else if (split) {
    S = (steps_total + kSplitSliceSteps - 1) / kSplitSliceSteps;
    if (M <= 4 && (N + 16 * kWaves - 1) / (16 * kWaves) * S >= kWideTileMinWgs) groups = 4;
  }
  p.rows_per_wg = 4 * groups * kWaves;
  p.row_tiles = (int)((N + p.rows_per_wg - 1) / p.rows_per_wg);
  if (split_k <= 0)
    while ((int64_t)S * p.row_tiles < kMinWgs && steps_total / (S + 1) >= 1) ++S;
  if (S < 1) S = 1;
  int sps = (steps_total + S - 1) / S;                 // steps per slice
  const int max_sps = groups == 2 ? max_pair_steps(M) : kMaxSliceSteps;
  if (sps > max_sps) sps = max_sps;
  if (sps < 1) sps = 1;
  p.blocks_per_split = sps * kStepBlocks;
  p.splits = (nb + p.blocks_per_split - 1) / p.blocks_per_split;
  if (p.splits > 1) {
    p.counter_bytes = kCounterRegionBytes;
    p.ws_bytes = p.counter_bytes + (size_t)p.splits * M * N * sizeof(float);
  }
  return p;
}

hipError_t launch_skinny_mfma4(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                               uint16_t* y, int M, int64_t N, int64_t K, const SkinnyPlan& p,
                               void* ws, hipStream_t s) {
  switch (M) {
    case 3: return launch_m<3>(x, codes, scales, y, N, K, p, ws, s);
    case 4: return launch_m<4>(x, codes, scales, y, N, K, p, ws, s);
    case 5: return launch_m<5>(x, codes, scales, y, N, K, p, ws, s);
    case 6: return launch_m<6>(x, codes, scales, y, N, K, p, ws, s);
    case 7: return launch_m<7>(x, codes, scales, y, N, K, p, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4w
