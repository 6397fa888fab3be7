// q4_gemv_skinny on the matrix cores, for the verify widths 4 <= M <= 8.
//
// The VALU form of the skinny matmul pays M/2 dot2 lane-ops per weight, which
// outgrows the HBM stream as M grows (speculative verification scores
// 1 + drafted tokens per pass: page 3, "Qwen3.8-27B at 256K on a 24GB RTX PRO
// 4000 SFF", the MTP n_max = 3 result; page 5, "Qwen3.8-27B on RTX 4090:
// 5,000 tok/s Prefill Reproduced", sections on MTP and DFlash2 windows).
// Here the M activation rows ride through v_mfma_f32_16x16x32_f16 instead, so
// the VALU work per weight is the unpack plus one scale FMA per block and no
// longer grows with M.
//
// 16x16x32 f16 MFMA, lane l, g = l / 16, c = l % 16:
//   A (16 x 32): lane l supplies 8 k-slots of row c (slot group g)
//   B (32 x 16): lane l supplies the same 8 k-slots of column c
//   D (16 x 16): lane l holds rows 4g .. 4g+3 of column c
// A = the activation rows (rows M..15 zero), B = 16 weight rows x one
// 32-weight block, so every column of one MFMA shares one block and the
// block's fp16 scale can be applied to D afterwards (one FMA per D row).
//
//  * Loads: lane (c, g) reads the 16-byte block 4s + g of its row, so one
//    128-bit load of a wave covers 16 rows x 64 contiguous bytes.  A 4x4
//    transpose across the lane groups (two permlane32 and two permlane16
//    swaps) then gives lane (c, g) word g of each of the 4 blocks, which is
//    exactly its B-operand share of each block's MFMA.
//  * Unpack as in the VALU kernel: one bit op per fp16 pair, (1024 + q + 8)
//    for even k and (64 + q + 8) for odd k; the MFMA starts from -bias of the
//    block (1032 sum x_even + 72 sum x_odd per activation row), staged in LDS
//    with the permuted activations.
//  * Split-K and its deterministic fixup as in the VALU kernel.

#include "q4w_internal.h"
#include "splitk.h"
#include <hip/hip_fp16.h>

namespace q4w {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kBlocksPerStep = 4;            // one 128-bit load per lane = 4 blocks per lane group set
constexpr int kLdsBytesPerBlock = 64 * 16 + 16 * 4;   // A octets for 64 lanes + 16 biases
constexpr int kMaxSliceSteps = 8;            // K-slice cap: 32 blocks, 34 KB of LDS
constexpr int kStageItems = kMaxSliceSteps * kBlocksPerStep * 16 / kThreads;   // (block, row) items per thread

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

// Lanes 32..63 of a <-> lanes 0..31 of b.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
// Lanes 16..31 and 48..63 of a <-> lanes 0..15 and 32..47 of b.
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// v[r] of lane group g holds word r of block g  ->  v[j] holds word g of block j.
__device__ __forceinline__ void transpose4(uint32_t (&v)[4]) {
  swap32(v[0], v[2]);
  swap32(v[1], v[3]);
  swap16(v[0], v[1]);
  swap16(v[2], v[3]);
}

}  // namespace

// Tiles of 16 rows per wave and steps in flight per wave.  Slices are at
// most one ring long, so every load of a slice is issued at once: on MI355X
// the stream only reaches full rate when each wave has all of its bytes in
// flight.
__host__ __device__ constexpr int mfma_tiles_per_wave(int) { return 1; }
__host__ __device__ constexpr int mfma_ring_steps(int) { return 8; }

namespace {

// kScaleQuad: K % 128 == 0, so the 4 scales of a step are one aligned 8-byte
// load (otherwise four 2-byte loads).
template <int M, bool kScaleQuad>
__global__ void __launch_bounds__(kThreads)
mfma_skinny_kernel(const uint16_t* __restrict__ x, const uint4* __restrict__ codes,
                   const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
                   float* __restrict__ partial, uint32_t* __restrict__ counters,
                   int N, int K, int bps, int S) {
  constexpr int R = mfma_tiles_per_wave(M);
  constexpr int P = mfma_ring_steps(M);
  constexpr int kRowsPerWg = kWaves * R * 16;
  constexpr int RM = M < 4 ? M : 4;          // D rows a lane accumulates
  extern __shared__ uint4 smem[];

  const int nb = K / kBlock;
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int kb0 = split * bps;
  const int nbs = min(bps, nb - kb0);
  const int steps = (nbs + kBlocksPerStep - 1) / kBlocksPerStep;
  const int bpad = steps * kBlocksPerStep;

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int tile_row0 = tile * kRowsPerWg;
  const int rows_here = min(kRowsPerWg, N - tile_row0);

  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + (size_t)tile_row0 * nb), 0, rows_here * nb * kBlockBytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + (size_t)tile_row0 * nb), 0, rows_here * nb * 2, kRsrcWord3);
  uint32_t vblk[R];    // tile-local block index of this lane's code load in step 0
  uint32_t vrow[R];    // tile-local index of block kb0 of this lane's row
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int rl = (wave * R + i) * 16 + col;
    vrow[i] = (uint32_t)(rl * nb + kb0);
    vblk[i] = vrow[i] + grp;
  }

  // P steps of loads: codes (one 128-bit load per tile) and the 4 block
  // scales of the step for this lane's row.
  uint4 buf[P][R];
  uint32_t sbuf[P][R][kBlocksPerStep];
  auto load_step = [&](int t, uint4 (&c)[R], uint32_t (&sc)[R][kBlocksPerStep]) {
    const bool live = t * kBlocksPerStep + grp < nbs;
    const bool slive = t * kBlocksPerStep < nbs;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t vo = live ? vblk[i] * kBlockBytes : kOutOfRange;
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, t * kBlocksPerStep * kBlockBytes, 0);
      c[i] = make_uint4(v[0], v[1], v[2], v[3]);
      // Scales past the slice end only meet zero activations and zero bias.
      const uint32_t so = slive ? vrow[i] * 2 : kOutOfRange;
      if (kScaleQuad) {
        const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rs, so, t * kBlocksPerStep * 2, 0);
        sc[i][0] = v2[0] & 0xFFFFu;
        sc[i][1] = v2[0] >> 16;
        sc[i][2] = v2[1] & 0xFFFFu;
        sc[i][3] = v2[1] >> 16;
      } else {
#pragma unroll
        for (int j = 0; j < kBlocksPerStep; ++j)
          sc[i][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, t * kBlocksPerStep * 2 + 2 * j, 0);
      }
    }
  };
  // ---- activation loads first: (block b, row m) items of this slice ------
  // Their data is needed before any weight step, and loads complete in issue
  // order, so they go out ahead of the weight loads.  Rows m >= M and blocks
  // past the slice read zeros (out-of-range offset, no memory request).
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, M * K * 2, kRsrcWord3);
  uint4 raw[kStageItems][4];
#pragma unroll
  for (int it = 0; it < kStageItems; ++it) {
    const int u = tid + it * kThreads;
    const int b = u >> 4;
    const int m = u & 15;
    const bool valid = m < M && b < nbs;
    const uint32_t xo = valid ? (uint32_t)(m * K + (kb0 + b) * kBlock) * 2 : kOutOfRange;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, q * 16, 0);
      raw[it][q] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }

#pragma unroll
  for (int p = 0; p < P; ++p) load_step(p, buf[p], sbuf[p]);

  // ---- stage A operands and biases: xs[b][g][m] (16 rows, M..15 zero) -----
  uint4* xs = smem;
  float* cl = reinterpret_cast<float*>(smem + bpad * 64);   // [bpad][16] -bias
  const uint32_t k1032 = 0x64086408u;
  const uint32_t k72 = 0x54805480u;
#pragma unroll
  for (int it = 0; it < kStageItems; ++it) {
    const int u = tid + it * kThreads;
    if (u < bpad * 16) {
      const int b = u >> 4;
      const int m = u & 15;
      float c = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // elements e0..e7 of code word q -> (e0,e4), (e1,e5), (e2,e6), (e3,e7)
        const uint32_t w0 = raw[it][q].x, w1 = raw[it][q].y, w2 = raw[it][q].z, w3 = raw[it][q].w;
        uint4 o;
        o.x = (w0 & 0xFFFFu) | (w2 << 16);
        o.y = (w0 >> 16) | (w2 & 0xFFFF0000u);
        o.z = (w1 & 0xFFFFu) | (w3 << 16);
        o.w = (w1 >> 16) | (w3 & 0xFFFF0000u);
        xs[b * 64 + q * 16 + m] = o;
        c = dot2(o.x, k1032, c);
        c = dot2(o.y, k72, c);
        c = dot2(o.z, k1032, c);
        c = dot2(o.w, k72, c);
      }
      cl[b * 16 + m] = -c;
    }
  }
  __syncthreads();

  f4 yacc[R];
#pragma unroll
  for (int i = 0; i < R; ++i) yacc[i] = f4{0.f, 0.f, 0.f, 0.f};

  auto compute_step = [&](int t, const uint4 (&c)[R], const uint32_t (&sc)[R][kBlocksPerStep]) {
    uint32_t w[R][4];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      w[i][0] = c[i].x;
      w[i][1] = c[i].y;
      w[i][2] = c[i].z;
      w[i][3] = c[i].w;
      transpose4(w[i]);
    }
    // All MFMAs of the step first, then their scale FMAs: the MFMA results
    // are independent, so their latencies overlap.
    f4 d4[kBlocksPerStep][R];
#pragma unroll
    for (int j = 0; j < kBlocksPerStep; ++j) {
      const int b = t * kBlocksPerStep + j;
      const uint4 av = xs[b * 64 + lane];
      const f4 cv = reinterpret_cast<const f4*>(cl)[b * 4 + grp];
      const h8 a = __builtin_bit_cast(h8, av);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const uint32_t u = w[i][j];
        const uint32_t u8 = u >> 8;
        v4u bw;
        bw[0] = (u & 0x000F000Fu) ^ 0x64086408u;    // (1024 + q + 8) at k0, k4
        bw[1] = (u & 0x00F000F0u) ^ 0x54805480u;    // (64 + q + 8)   at k1, k5
        bw[2] = (u8 & 0x000F000Fu) ^ 0x64086408u;   // k2, k6
        bw[3] = (u8 & 0x00F000F0u) ^ 0x54805480u;   // k3, k7
        d4[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(h8, bw), cv, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < kBlocksPerStep; ++j)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float s = __half2float(__ushort_as_half((unsigned short)sc[i][j]));
#pragma unroll
        for (int r = 0; r < RM; ++r) yacc[i][r] = fmaf(d4[j][i][r], s, yacc[i][r]);
      }
  };

  // A slice is at most P steps (the plan guarantees it): no refills.
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < steps) compute_step(p, buf[p], sbuf[p]);

  // ---- store: lane (col, grp) holds rows 4 grp + r of its column ---------
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int n = tile_row0 + (wave * R + i) * 16 + col;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const int m = 4 * grp + r;
      if (m < M && n < N) {
        if (S == 1) y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(yacc[i][r]));
        else
          __hip_atomic_store(&partial[((size_t)split * M + m) * N + n], yacc[i][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
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
  for (int o = tid; o < kRowsPerWg * M; o += kThreads) {
    const int m = o / kRowsPerWg;
    const int n = tile_row0 + (o - m * kRowsPerWg);
    if (n < N) {
      const float s = sum_partials(&partial[(size_t)m * N + n], (size_t)M * N, S);
      y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(s));
    }
  }
  if (tid == 0)
    __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int M>
hipError_t launch_mfma_m(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                         uint16_t* y, int64_t N, int64_t K, const SkinnyPlan& p, void* ws,
                         hipStream_t s) {
  const int bpad = ((p.blocks_per_split + kBlocksPerStep - 1) / kBlocksPerStep) * kBlocksPerStep;
  const size_t lds = (size_t)bpad * kLdsBytesPerBlock;
  uint32_t* counters = nullptr;
  float* partial = nullptr;
  if (p.splits > 1) {
    counters = reinterpret_cast<uint32_t*>(ws);
    partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.counter_bytes);
  }
  const bool quad = (K / kBlock) % kBlocksPerStep == 0;
  const dim3 grid(p.row_tiles, p.splits);
  const uint4* c4 = reinterpret_cast<const uint4*>(codes);
  const int n = (int)N, k = (int)K, bps = p.blocks_per_split, S = p.splits;
  if (quad)
    hipLaunchKernelGGL((mfma_skinny_kernel<M, true>), grid, dim3(kThreads), lds, s, x, c4,
                       scales, y, partial, counters, n, k, bps, S);
  else
    hipLaunchKernelGGL((mfma_skinny_kernel<M, false>), grid, dim3(kThreads), lds, s, x, c4,
                       scales, y, partial, counters, n, k, bps, S);
  return hipGetLastError();
}

}  // namespace

// Split plan of the matrix-core kernel: slices are whole 4-block steps, at
// most one ring (kMaxSliceSteps) long, with enough slices to put about four
// workgroups on every CU.
SkinnyPlan plan_skinny_mfma(int M, int64_t N, int64_t K, int split_k) {
  SkinnyPlan p{};
  p.route = kRouteMfma;
  p.rows_per_wg = kWaves * mfma_tiles_per_wave(M) * 16;
  p.row_tiles = (int)((N + p.rows_per_wg - 1) / p.rows_per_wg);
  const int nb = (int)(K / kBlock);
  const int steps_total = (nb + kBlocksPerStep - 1) / kBlocksPerStep;
  static_assert(kMaxSliceSteps <= mfma_ring_steps(0), "a slice fits the ring");
  const int lds_steps = kMaxSliceSteps;
  int steps;
  if (split_k > 0) {
    steps = (steps_total + split_k - 1) / split_k;
    if (steps > lds_steps) steps = lds_steps;
  } else {
    int max_steps = lds_steps;
    int S = (steps_total + max_steps - 1) / max_steps;
    const int target_wgs = 1024;
    while ((int64_t)S * p.row_tiles < target_wgs && steps_total / (S + 1) >= 2) ++S;
    steps = (steps_total + S - 1) / S;
  }
  if (steps < 1) steps = 1;
  p.blocks_per_split = steps * kBlocksPerStep;
  p.splits = (nb + p.blocks_per_split - 1) / p.blocks_per_split;
  if (p.splits > 1) {
    p.counter_bytes = kCounterRegionBytes;
    p.ws_bytes = p.counter_bytes + (size_t)p.splits * M * N * sizeof(float);
  }
  return p;
}

hipError_t launch_skinny_mfma(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                              uint16_t* y, int M, int64_t N, int64_t K, const SkinnyPlan& p,
                              void* ws, hipStream_t s) {
  switch (M) {
    case 4: return launch_mfma_m<4>(x, codes, scales, y, N, K, p, ws, s);
    case 5: return launch_mfma_m<5>(x, codes, scales, y, N, K, p, ws, s);
    case 6: return launch_mfma_m<6>(x, codes, scales, y, N, K, p, ws, s);
    case 7: return launch_mfma_m<7>(x, codes, scales, y, N, K, p, ws, s);
    case 8: return launch_mfma_m<8>(x, codes, scales, y, N, K, p, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4w
