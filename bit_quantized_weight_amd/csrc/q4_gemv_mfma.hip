// q4_gemv_skinny on the matrix cores, for the verify widths 4 <= M <= 16.
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

#include <algorithm>
#include <functional>
#include <queue>
#include <utility>
#include <vector>

// Streaming kernel shape (measured best on the 64-layer decode step at M = 1
// and 5): 8-step chunks, 3 waves per SIMD, 4 row tiles per work item.
#ifndef STREAM_P
#define STREAM_P 8
#endif
#ifndef STREAM_WAVES
#define STREAM_WAVES 3
#endif
#ifndef STREAM_TILES
#define STREAM_TILES 4
#endif

namespace q4w {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Split-K fixup: partial loads in flight per thread.  A 64-row tile at M <= 8
// has at most 2 outputs per thread, so S <= 18 slices take one round.
constexpr int kFixupBatch = 36;
constexpr int kMinMfmaWgs = 256;             // one workgroup per CU
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kBlocksPerStep = 4;            // one 128-bit load per lane = 4 blocks per lane group set
constexpr int kMaxSliceSteps = 8;            // K-slice cap: 32 blocks
// Row map of the products.  Lane group g holds D rows 4 g .. 4 g + 3 and
// applies the block scale to each of them that holds an activation row.  Up
// to M = 8, activation row m is row mfma_row = 4 (m % 4) + m / 4 of A and D
// (a 4 x 4 transpose of the row index, its own inverse): group g holds rows
// g, g + 4 of the activations, so a lane scales d_rows = ceil(M / 4) D rows
// (one at M <= 4, where rows 0..3 in order would take min(M, 4)).  Past
// M = 8 the rows stay in order (four D rows per lane either way).  Row r of
// a product depends on A row r only, so any row map gives the same values.
__host__ __device__ constexpr bool rows_transposed(int M) { return M <= 8; }
__host__ __device__ constexpr int mfma_row(int M, int m) {
  return rows_transposed(M) ? 4 * (m & 3) + (m >> 2) : m;
}
__host__ __device__ constexpr int d_rows(int M) { return rows_transposed(M) ? (M + 3) / 4 : 4; }
// Lane group g's D rows hold at least one activation row.
__host__ __device__ constexpr bool group_live(int M, int g) { return rows_transposed(M) ? g < M : 4 * g < M; }
// Activation row held by D row r of lane group g.
__host__ __device__ constexpr int act_row(int M, int g, int r) { return rows_transposed(M) ? g + 4 * r : 4 * g + r; }
// -bias floats per block, indexed by MFMA row: lane group g reads rows
// 4 g .. 4 g + 3 (at M = 1 only group 0 has a real row).
__host__ __device__ constexpr int bias_slots(int M) { return M == 1 ? 4 : rows_transposed(M) ? 16 : (M + 3) / 4 * 4; }
// LDS per block of the slice: the M activation rows as A-operand octets
// (4 slot groups x M rows x 16 bytes) and the -bias of each MFMA row that
// holds an activation (the other slots are never written: the D rows they
// start are never stored).  A-operand rows that hold no activation are not
// stored either: their lanes read activation row 0's octets instead, which
// keeps each LDS address a per-lane base plus a constant offset.
__host__ __device__ constexpr int mp4(int M) { return (M + 3) / 4 * 4; }
__host__ __device__ constexpr int lds_bytes_per_block(int M) { return 64 * M + 4 * bias_slots(M); }
// Steps of a K-chunk whose (block, row) staging items fit kItems per thread,
// at most kMaxSliceSteps.  The streaming kernel stages one item per thread;
// the single-launch kernel up to two (8 steps for every M <= 16).
__host__ __device__ constexpr int chunk_steps(int M, int items) {
  return items * kThreads / (kBlocksPerStep * mp4(M)) < kMaxSliceSteps
             ? items * kThreads / (kBlocksPerStep * mp4(M))
             : kMaxSliceSteps;
}
__host__ __device__ constexpr int max_slice_steps(int M) { return chunk_steps(M, 2); }
__host__ __device__ constexpr int stage_items(int M) {
  return (max_slice_steps(M) * kBlocksPerStep * mp4(M) + kThreads - 1) / kThreads;
}
__host__ __device__ constexpr int lds_bytes(int M, int bpad) { return bpad * lds_bytes_per_block(M); }

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

// One work item: row tile `tile` (64 rows) x K-slice `split` of one matmul.
// kScaleQuad: K % 128 == 0, so the 4 scales of a step are one aligned 8-byte
// load (otherwise four 2-byte loads).  The LDS of the previous item of this
// workgroup is overwritten only after a barrier.
template <int M, bool kScaleQuad>
__device__ __forceinline__ void mfma_item(const uint16_t* __restrict__ x,
                                          const uint4* __restrict__ codes,
                                          const uint16_t* __restrict__ scales,
                                          uint16_t* __restrict__ y, float* __restrict__ partial,
                                          uint32_t* __restrict__ counters, int N, int K, int bps,
                                          int S, int tile, int split, uint4* smem) {
  constexpr int R = mfma_tiles_per_wave(M);
  constexpr int P = mfma_ring_steps(M);
  constexpr int kRowsPerWg = kWaves * R * 16;
  constexpr int RM = d_rows(M);              // D rows a lane accumulates

  const int nb = K / kBlock;
  const int tid = threadIdx.x;
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
  // Item u = tid + it * kThreads is (block u / Mp4, row u % Mp4):
  // bpad x Mp4 <= kItems x kThreads items (one per thread up to M = 8).
  constexpr int MP = mp4(M);
  constexpr int kItems = stage_items(M);
  static_assert(max_slice_steps(M) * kBlocksPerStep * MP <= kItems * kThreads, "staging items");
  uint4 raw[kItems][4];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int u = tid + it * kThreads;
    const int sb = u / MP, sm = u % MP;
    const bool valid = sm < M && sb < nbs;
    const uint32_t xo = valid ? (uint32_t)(sm * K + (kb0 + sb) * kBlock) * 2 : kOutOfRange;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, q * 16, 0);
      raw[it][q] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }

#pragma unroll
  for (int p = 0; p < P; ++p) load_step(p, buf[p], sbuf[p]);

  // ---- stage A operands and biases: xs[b][g][m] (m < M), cl[b][mfma_row(m)] -
  __syncthreads();   // the previous item of this workgroup is done with the LDS
  char* lds = reinterpret_cast<char*>(smem);
  uint4* xs = smem;                                                    // [bpad][4][M]
  float* cl = reinterpret_cast<float*>(lds + bpad * 64 * M);           // [bpad][bias_slots]
  const uint32_t k1032 = 0x64086408u;
  const uint32_t k72 = 0x54805480u;
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int u = tid + it * kThreads;
    const int sb = u / MP, sm = u % MP;
    if (sb < bpad) {
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
        if (sm < M) xs[(sb * 4 + q) * M + sm] = o;
        c = dot2(o.x, k1032, c);
        c = dot2(o.y, k72, c);
        c = dot2(o.z, k1032, c);
        c = dot2(o.w, k72, c);
      }
      if (sm < M) cl[sb * bias_slots(M) + mfma_row(M, sm)] = -c;
    }
  }
  __syncthreads();

  // Per-lane LDS addresses: A octet of block b at a_base + b * a_stride
  // (MFMA rows without an activation read row 0's), bias float4 of MFMA rows
  // 4 grp.. at c_base + b * c_stride (groups without a real row read group
  // 0's).  The strides are constants, so the compiler folds b * stride into
  // the LDS instruction.
  const int am = mfma_row(M, col);
  const int a_base = (grp * M + (am < M ? am : 0)) * 16;
  constexpr int a_stride = 64 * M;
  const int c_base = bpad * 64 * M + (group_live(M, grp) ? grp : 0) * 16;
  constexpr int c_stride = bias_slots(M) * 4;

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
      const uint4 av = *reinterpret_cast<const uint4*>(lds + a_base + b * a_stride);
      const f4 cv = *reinterpret_cast<const f4*>(lds + c_base + b * c_stride);
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

  // ---- store: lane (col, grp) holds activation rows act_row(grp, r) -------
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int n = tile_row0 + (wave * R + i) * 16 + col;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      const int m = act_row(M, grp, r);
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
  fixup_tile<kRowsPerWg, M, kThreads, kFixupBatch>(partial, y, N, S, tile_row0);
  if (tid == 0)
    __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Occupancy floor: with 6 waves per SIMD (at most 80 VGPRs) every workgroup
// of a 1024..1536-workgroup split plan is resident at once, so no second
// partial wave of workgroups trails the stream.  Two staging items per
// thread (M > 8) and the four-load scale form need more registers and take
// what fits without spilling.
template <int M, bool kScaleQuad>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kScaleQuad ? (stage_items(M) > 1 ? 5 : 6) : (stage_items(M) > 1 ? 4 : 5), 8)))
mfma_skinny_kernel(const uint16_t* __restrict__ x, const uint4* __restrict__ codes,
                   const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
                   float* __restrict__ partial, uint32_t* __restrict__ counters,
                   int N, int K, int bps, int S) {
  extern __shared__ uint4 smem[];
  mfma_item<M, kScaleQuad>(x, codes, scales, y, partial, counters, N, K, bps, S, blockIdx.x,
                           blockIdx.y, smem);
}

// Streaming form: one persistent launch computes every matmul of a table
// (same M).  A work item is kStreamTiles row tiles of 64 rows over the whole
// of K (no split-K: no partials, no arrival counters, no waits on store
// completion).  A workgroup walks its own list of items (dealt at plan time
// so that every workgroup gets about the same rows x K) as a sequence
// of units (K-chunk c, tile t), tile innermost: the activations of chunk c
// are staged into LDS once (one barrier) and serve all tiles of the item.
// The loads of the next unit (codes, scales, and activations at tile 0) go
// into the other register set before the current unit is computed, so each
// wave keeps a chunk of weights in flight while it stages and computes.
// Two LDS activation buffers alternate by chunk.
// Steps per chunk of the streaming kernel (two chunks of loads stay in
// registers) and 64-row tiles per work item.
__host__ __device__ constexpr int stream_steps(int M, bool quad) {
  return !quad ? 4 : (chunk_steps(M, 1) / 4 * 4 < STREAM_P ? chunk_steps(M, 1) / 4 * 4 : STREAM_P);
}
constexpr int kStreamTiles = STREAM_TILES;

struct Walker {
  int pos;       // position in this workgroup's item list
  int next;      // the item at pos + 1 (read ahead)
  int item;      // work item of matmul g
  int g;         // matmul index
  int chunk;     // chunk along K
  int tile;      // tile within the item
  int nchunks;   // chunks of this matmul
  bool valid;
};

template <int M, bool kScaleQuad>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(STREAM_WAVES, 8)))
mfma_stream_kernel(const BatchedGemv* __restrict__ table, int count, const uint32_t* __restrict__ sched) {
  constexpr int P = stream_steps(M, kScaleQuad);
  constexpr int T = kStreamTiles;
  constexpr int kChunkBlocks = P * kBlocksPerStep;
  constexpr int MP = mp4(M);
  constexpr int RM = d_rows(M);
  constexpr int kLdsBuf = lds_bytes(M, kChunkBlocks);
  constexpr int kSets = 2;
  static_assert(T % kSets == 0, "units cycle through register sets and tiles together");
  extern __shared__ uint4 smem[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int sb = tid / MP;                 // staging block of this thread
  const int sm = tid % MP;                 // staging row of this thread
  const int rl = wave * 16 + col;          // tile-local weight row of this lane

  // Per-lane LDS addresses (see mfma_item), for a buffer of kChunkBlocks blocks.
  const int am = mfma_row(M, col);
  const int a_base = (grp * M + (am < M ? am : 0)) * 16;
  constexpr int a_stride = 64 * M;
  const int c_base = kChunkBlocks * 64 * M + (group_live(M, grp) ? grp : 0) * 16;
  constexpr int c_stride = bias_slots(M) * 4;

  // This workgroup's items, ascending: items[pos] for pos in [first, end).
  const uint32_t* items = sched + (kMaxBatchedGrid + 1);
  const int end = (int)sched[blockIdx.x + 1];
  auto start = [&](Walker& w, int pos, int item) {
    w.pos = pos;
    w.item = item;
    w.valid = pos < end;
    if (!w.valid) return;
    w.next = pos + 1 < end ? (int)items[pos + 1] : 0;
    while (w.g + 1 < count && item >= table[w.g + 1].item_begin) ++w.g;
    w.chunk = 0;
    w.tile = 0;
    w.nchunks = (table[w.g].K / kBlock + kChunkBlocks - 1) / kChunkBlocks;
  };
  auto advance = [&](const Walker& w) {
    Walker n = w;
    if (w.tile + 1 < T) {
      ++n.tile;
    } else if (w.chunk + 1 < w.nchunks) {
      ++n.chunk;
      n.tile = 0;
    } else {
      start(n, w.pos + 1, w.next);
    }
    return n;
  };

  // One register set: a unit's codes and scales.  Scales with kScaleQuad:
  // lane group g loads the 4 scales of step 4l + g of its row (8 bytes), one
  // load per 4 steps; the groups' words are all-gathered with permlane swaps
  // at compute time.  Otherwise four 2-byte loads per step.  The scales are
  // requested before the codes, so the first step's products and scale FMAs
  // wait for its own codes only, not for the whole unit.
  static_assert(P % kBlocksPerStep == 0, "scale loads cover 4 steps each");
  constexpr int kScaleLoads = P / kBlocksPerStep;
  struct Set {
    uint4 w[P];
    uint32_t s[kScaleQuad ? kScaleLoads : P][kScaleQuad ? 2 : kBlocksPerStep];
  };
  // This thread's activation item of the next chunk (loaded with the chunk's
  // tile-0 unit, consumed when that chunk is staged).
  uint4 xbuf[4];
  auto issue = [&](const Walker& w, Set& st, bool with_x) {
    const BatchedGemv& d = table[w.valid ? w.g : 0];
    const int nb = d.K / kBlock;
    const int kb0 = w.chunk * kChunkBlocks;
    const int nbs = w.valid ? min(kChunkBlocks, nb - kb0) : 0;
    const int tile_row0 = ((w.item - d.item_begin) * T + w.tile) * 64;
    const int rows_here = w.valid ? max(0, min(64, d.N - tile_row0)) : 0;
    const size_t row0 = rows_here > 0 ? (size_t)tile_row0 : 0;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(d.codes + row0 * nb), 0, rows_here * nb * kBlockBytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(d.scales + row0 * nb), 0, rows_here * nb * 2, kRsrcWord3);
    if (with_x) {
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          (void*)d.x, 0, w.valid ? M * d.K * 2 : 0, kRsrcWord3);
      const bool valid = sm < M && sb < nbs;
      const uint32_t xo = valid ? (uint32_t)(sm * d.K + (kb0 + sb) * kBlock) * 2 : kOutOfRange;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, q * 16, 0);
        xbuf[q] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
    const uint32_t vrow = (uint32_t)(rl * nb + kb0);
    if constexpr (kScaleQuad) {
#pragma unroll
      for (int l = 0; l < kScaleLoads; ++l) {
        const int t = l * kBlocksPerStep + grp;     // the step whose scales this lane loads
        const uint32_t so = t * kBlocksPerStep < nbs ? (vrow + t * kBlocksPerStep) * 2 : kOutOfRange;
        const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rs, so, 0, 0);
        st.s[l][0] = v2[0];
        st.s[l][1] = v2[1];
      }
    } else {
#pragma unroll
      for (int t = 0; t < P; ++t) {
        const uint32_t so = t * kBlocksPerStep < nbs ? vrow * 2 : kOutOfRange;
#pragma unroll
        for (int j = 0; j < kBlocksPerStep; ++j)
          st.s[t][j] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, t * kBlocksPerStep * 2 + 2 * j, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < P; ++t) {
      const bool live = t * kBlocksPerStep + grp < nbs;
      const uint32_t vo = live ? (vrow + grp) * kBlockBytes : kOutOfRange;
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, t * kBlocksPerStep * kBlockBytes, 0);
      st.w[t] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  // Value of lane group g's v in every lane: out[g].
  auto all_gather4 = [](uint32_t v, uint32_t (&out)[4]) {
    uint32_t x = v, y = v;
    swap32(x, y);            // x: groups (0, 1, 0, 1), y: (2, 3, 2, 3)
    uint32_t a = x, b = x, c = y, e = y;
    swap16(a, b);            // a: group 0 everywhere, b: group 1
    swap16(c, e);            // c: group 2, e: group 3
    out[0] = a;
    out[1] = b;
    out[2] = c;
    out[3] = e;
  };

  // stage a chunk's activations into an LDS buffer (blocks past it are zeros)
  auto stage = [&](char* lds) {
    if (sb < kChunkBlocks) {
      uint4* xs = reinterpret_cast<uint4*>(lds);
      float* cl = reinterpret_cast<float*>(lds + kChunkBlocks * 64 * M);
      float c = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w0 = xbuf[q].x, w1 = xbuf[q].y, w2 = xbuf[q].z, w3 = xbuf[q].w;
        uint4 o;
        o.x = (w0 & 0xFFFFu) | (w2 << 16);
        o.y = (w0 >> 16) | (w2 & 0xFFFF0000u);
        o.z = (w1 & 0xFFFFu) | (w3 << 16);
        o.w = (w1 >> 16) | (w3 & 0xFFFF0000u);
        if (sm < M) xs[(sb * 4 + q) * M + sm] = o;
        c = dot2(o.x, 0x64086408u, c);
        c = dot2(o.y, 0x54805480u, c);
        c = dot2(o.z, 0x64086408u, c);
        c = dot2(o.w, 0x54805480u, c);
      }
      if (sm < M) cl[sb * bias_slots(M) + mfma_row(M, sm)] = -c;
    }
  };

  // compute a unit into one tile's accumulators; store them after the last chunk
  auto compute = [&](const Walker& w, const Set& st, const char* lds, f4& yacc) {
    const BatchedGemv& d = table[w.g];
    const int nb = d.K / kBlock;
    const int nbs = min(kChunkBlocks, nb - w.chunk * kChunkBlocks);
    const int steps = (nbs + kBlocksPerStep - 1) / kBlocksPerStep;
    // scales of step t, block j: quad -> word (j >> 1) of lane group (t % 4)
    // of load t / 4, half (j & 1)
    uint32_t sg[kScaleQuad ? kScaleLoads : 1][2][4];
    if constexpr (kScaleQuad) {
#pragma unroll
      for (int l = 0; l < kScaleLoads; ++l) {
        all_gather4(st.s[l][0], sg[l][0]);
        all_gather4(st.s[l][1], sg[l][1]);
      }
    }
    auto scale_of = [&](int t, int j) -> float {
      uint32_t bits;
      if constexpr (kScaleQuad) {
        const uint32_t wd = sg[t / kBlocksPerStep][j >> 1][t % kBlocksPerStep];
        bits = (j & 1) ? (wd >> 16) : (wd & 0xFFFFu);
      } else {
        bits = st.s[t][j];
      }
      return __half2float(__ushort_as_half((unsigned short)bits));
    };
#pragma unroll
    for (int t = 0; t < P; ++t) {
      if (t < steps) {
        uint32_t wv[4] = {st.w[t].x, st.w[t].y, st.w[t].z, st.w[t].w};
        transpose4(wv);
        f4 d4[kBlocksPerStep];
#pragma unroll
        for (int j = 0; j < kBlocksPerStep; ++j) {
          const int b = t * kBlocksPerStep + j;
          const h8 a = __builtin_bit_cast(h8, *reinterpret_cast<const uint4*>(lds + a_base + b * a_stride));
          const f4 cv = *reinterpret_cast<const f4*>(lds + c_base + b * c_stride);
          const uint32_t u = wv[j];
          const uint32_t u8 = u >> 8;
          v4u bw;
          bw[0] = (u & 0x000F000Fu) ^ 0x64086408u;
          bw[1] = (u & 0x00F000F0u) ^ 0x54805480u;
          bw[2] = (u8 & 0x000F000Fu) ^ 0x64086408u;
          bw[3] = (u8 & 0x00F000F0u) ^ 0x54805480u;
          d4[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(h8, bw), cv, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kBlocksPerStep; ++j) {
          const float sc = scale_of(t, j);
#pragma unroll
          for (int r = 0; r < RM; ++r) yacc[r] = fmaf(d4[j][r], sc, yacc[r]);
        }
      }
    }
    if (w.chunk + 1 == w.nchunks) {          // this tile is done: store its 64 x M outputs
      const int n = ((w.item - d.item_begin) * T + w.tile) * 64 + rl;
#pragma unroll
      for (int r = 0; r < RM; ++r) {
        const int m = act_row(M, grp, r);
        if (m < M && n < d.N) d.y[(size_t)m * d.N + n] = __half_as_ushort(__float2half_rn(yacc[r]));
      }
      yacc = f4{0.f, 0.f, 0.f, 0.f};
    }
  };

  char* lds0 = reinterpret_cast<char*>(smem);

  Set sets[kSets];
  Walker w[kSets];
  f4 yacc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) yacc[t] = f4{0.f, 0.f, 0.f, 0.f};
  w[0] = Walker{};
  {
    const int first = (int)sched[blockIdx.x];
    start(w[0], first, first < end ? (int)items[first] : 0);
  }
  issue(w[0], sets[0], true);
#pragma unroll
  for (int i = 1; i < kSets; ++i) {
    w[i] = advance(w[i - 1]);
    issue(w[i], sets[i], i % T == 0);
  }
  // Units arrive tile 0, 1, ..., T-1 per chunk, so unit u of each round of
  // T units is tile u and uses register set u % kSets (all static).
  int parity = 1;
  while (w[0].valid) {
#pragma unroll
    for (int u = 0; u < T; ++u) {
      Walker& cw = w[u % kSets];
      if (cw.valid) {
        if (u == 0) {                        // a new chunk: stage its activations
          parity ^= 1;
          stage(lds0 + parity * kLdsBuf);
          __syncthreads();
        }
        compute(cw, sets[u % kSets], lds0 + parity * kLdsBuf, yacc[u]);
        const Walker nw = advance(w[(u + kSets - 1) % kSets]);
        // the unit's loads go out at raised wave priority, ahead of the
        // other waves' arithmetic on this SIMD (-0.3 to -0.8% per step)
        __builtin_amdgcn_s_setprio(2);
        issue(nw, sets[u % kSets], (u + kSets) % T == 0);   // tile 0 of the next chunk
        __builtin_amdgcn_s_setprio(0);
        cw = nw;
      }
    }
  }
}

template <int M>
hipError_t launch_mfma_m(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                         uint16_t* y, int64_t N, int64_t K, const SkinnyPlan& p, void* ws,
                         hipStream_t s) {
  const int bpad = ((p.blocks_per_split + kBlocksPerStep - 1) / kBlocksPerStep) * kBlocksPerStep;
  const size_t lds = (size_t)lds_bytes(M, bpad);
  uint32_t* counters = nullptr;
  float* partial = nullptr;
  if (p.splits > 1) {
    counters = reinterpret_cast<uint32_t*>(ws);
    partial = reinterpret_cast<float*>(static_cast<char*>(ws) + p.counter_bytes);
  }
  const bool quad = (K / kBlock) % kBlocksPerStep == 0 && ((uintptr_t)scales & 7) == 0;
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
// most one ring (kMaxSliceSteps) long, so S is at least steps / 8.  More
// slices are added only below kMinMfmaWgs workgroups: the split-K fixup chain
// costs more than the extra parallelism buys (out 5120 -> 5120 at M = 5:
// 10 slices 9.8 us, 5 slices 8.9 us).
SkinnyPlan plan_skinny_mfma(int M, int64_t N, int64_t K, int split_k) {
  SkinnyPlan p{};
  p.route = kRouteMfma;
  p.rows_per_wg = kWaves * mfma_tiles_per_wave(M) * 16;
  p.row_tiles = (int)((N + p.rows_per_wg - 1) / p.rows_per_wg);
  const int nb = (int)(K / kBlock);
  const int steps_total = (nb + kBlocksPerStep - 1) / kBlocksPerStep;
  static_assert(kMaxSliceSteps <= mfma_ring_steps(0), "a slice fits the ring");
  const int lds_steps = max_slice_steps(M);
  int steps;
  if (split_k > 0) {
    steps = (steps_total + split_k - 1) / split_k;
    if (steps > lds_steps) steps = lds_steps;
  } else {
    int max_steps = lds_steps;
    int S = (steps_total + max_steps - 1) / max_steps;
    while ((int64_t)S * p.row_tiles < kMinMfmaWgs && steps_total / (S + 1) >= 1) ++S;
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

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// The streaming kernel's work items: kStreamTiles 64-row tiles over the whole of K.
static int64_t stream_tiles(int64_t N) { return (N + 64 * kStreamTiles - 1) / (64 * kStreamTiles); }

BatchedLayout batched_layout(int /*M*/, int count, const int64_t* N, const int64_t* /*K*/) {
  BatchedLayout L{};
  for (int g = 0; g < count; ++g) L.total_items += stream_tiles(N[g]);
  L.table_bytes = align256((size_t)count * sizeof(BatchedGemv));
  L.sched_bytes = align256(((size_t)kMaxBatchedGrid + 1 + (size_t)L.total_items) * sizeof(uint32_t));
  L.total_bytes = L.table_bytes + L.sched_bytes;
  return L;
}

void batched_schedule(int count, const int64_t* N, const int64_t* K, int grid, uint32_t* sched) {
  struct Item { int64_t cost; uint32_t index; };
  std::vector<Item> all;
  for (int g = 0, item = 0; g < count; ++g) {
    const int64_t tiles = stream_tiles(N[g]);
    for (int64_t t = 0; t < tiles; ++t, ++item) {
      const int64_t rows = std::min<int64_t>(64 * kStreamTiles, N[g] - t * 64 * kStreamTiles);
      all.push_back(Item{rows * K[g], (uint32_t)item});
    }
  }
  std::stable_sort(all.begin(), all.end(), [](const Item& a, const Item& b) { return a.cost > b.cost; });
  typedef std::pair<int64_t, int> Load;   // (assigned cost, workgroup)
  std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
  for (int w = 0; w < grid; ++w) heap.push(Load{0, w});
  std::vector<std::vector<uint32_t>> lists(grid);
  for (const Item& it : all) {
    Load l = heap.top();
    heap.pop();
    lists[l.second].push_back(it.index);
    l.first += it.cost;
    heap.push(l);
  }
  uint32_t* off = sched;
  uint32_t* items = sched + kMaxBatchedGrid + 1;
  uint32_t pos = 0;
  for (int w = 0; w < grid; ++w) {
    std::sort(lists[w].begin(), lists[w].end());
    off[w] = pos;
    for (uint32_t i : lists[w]) items[pos++] = i;
  }
  for (int w = grid; w <= kMaxBatchedGrid; ++w) off[w] = pos;
}

void batched_fill_table(int /*M*/, int count, const uint16_t* const* x,
                        const uint8_t* const* codes, const uint16_t* const* scales,
                        uint16_t* const* y, const int64_t* N, const int64_t* K, void* /*ws*/,
                        BatchedGemv* table) {
  int64_t item = 0;
  for (int g = 0; g < count; ++g) {
    BatchedGemv& d = table[g];
    d = BatchedGemv{};
    d.x = x[g];
    d.codes = reinterpret_cast<const uint4*>(codes[g]);
    d.scales = scales[g];
    d.y = y[g];
    d.N = (int)N[g];
    d.K = (int)K[g];
    d.bps = (int)(K[g] / kBlock);
    d.S = 1;
    d.item_begin = (int)item;
    item += stream_tiles(N[g]);
  }
}

namespace {
template <int M>
const void* batched_kernel_ptr(bool quad) {
  return quad ? reinterpret_cast<const void*>(&mfma_stream_kernel<M, true>)
              : reinterpret_cast<const void*>(&mfma_stream_kernel<M, false>);
}

// LDS of the streaming kernel: two chunk buffers.
int batched_lds(int M, bool quad) { return 2 * lds_bytes(M, stream_steps(M, quad) * kBlocksPerStep); }

const void* batched_kernel_for(int M, bool quad) {
  switch (M) {
    case 1: return batched_kernel_ptr<1>(quad);
    case 2: return batched_kernel_ptr<2>(quad);
    case 3: return batched_kernel_ptr<3>(quad);
    case 4: return batched_kernel_ptr<4>(quad);
    case 5: return batched_kernel_ptr<5>(quad);
    case 6: return batched_kernel_ptr<6>(quad);
    case 7: return batched_kernel_ptr<7>(quad);
    case 8: return batched_kernel_ptr<8>(quad);
    case 9: return batched_kernel_ptr<9>(quad);
    case 10: return batched_kernel_ptr<10>(quad);
    case 11: return batched_kernel_ptr<11>(quad);
    case 12: return batched_kernel_ptr<12>(quad);
    case 13: return batched_kernel_ptr<13>(quad);
    case 14: return batched_kernel_ptr<14>(quad);
    case 15: return batched_kernel_ptr<15>(quad);
    case 16: return batched_kernel_ptr<16>(quad);
    default: return nullptr;
  }
}
}  // namespace

bool batched_quad(int count, const int64_t* K, const uint16_t* const* scales) {
  for (int g = 0; g < count; ++g)
    if ((K[g] / kBlock) % kBlocksPerStep != 0 || ((uintptr_t)scales[g] & 7) != 0) return false;
  return true;
}

int batched_grid(int M, bool quad, int64_t total_items) {
  const void* k = batched_kernel_for(M, quad);
  int per_cu = 0, cus = 0, dev = 0;
  if (!k || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kThreads, batched_lds(M, quad)) != hipSuccess)
    return 0;
  int64_t grid = (int64_t)per_cu * cus;
  if (grid > total_items) grid = total_items;
  if (grid > kMaxBatchedGrid) grid = kMaxBatchedGrid;
  return (int)(grid < 1 ? 1 : grid);
}

hipError_t launch_batched(int M, bool quad, const void* ws, int count, int total_items,
                          int grid, hipStream_t s) {
  const void* k = batched_kernel_for(M, quad);
  if (!k) return hipErrorInvalidValue;
  const BatchedGemv* table = static_cast<const BatchedGemv*>(ws);
  const uint32_t* sched = reinterpret_cast<const uint32_t*>(
      static_cast<const char*>(ws) + align256((size_t)count * sizeof(BatchedGemv)));
  (void)total_items;
  void* args[] = {(void*)&table, (void*)&count, (void*)&sched};
  return hipLaunchKernel(k, dim3(grid), dim3(kThreads), args, batched_lds(M, quad), s);
}

hipError_t launch_skinny_mfma(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                              uint16_t* y, int M, int64_t N, int64_t K, const SkinnyPlan& p,
                              void* ws, hipStream_t s) {
  switch (M) {
    case 5: return launch_mfma_m<5>(x, codes, scales, y, N, K, p, ws, s);
    case 6: return launch_mfma_m<6>(x, codes, scales, y, N, K, p, ws, s);
    case 7: return launch_mfma_m<7>(x, codes, scales, y, N, K, p, ws, s);
    case 8: return launch_mfma_m<8>(x, codes, scales, y, N, K, p, ws, s);
    case 9: return launch_mfma_m<9>(x, codes, scales, y, N, K, p, ws, s);
    case 10: return launch_mfma_m<10>(x, codes, scales, y, N, K, p, ws, s);
    case 11: return launch_mfma_m<11>(x, codes, scales, y, N, K, p, ws, s);
    case 12: return launch_mfma_m<12>(x, codes, scales, y, N, K, p, ws, s);
    case 13: return launch_mfma_m<13>(x, codes, scales, y, N, K, p, ws, s);
    case 14: return launch_mfma_m<14>(x, codes, scales, y, N, K, p, ws, s);
    case 15: return launch_mfma_m<15>(x, codes, scales, y, N, K, p, ws, s);
    case 16: return launch_mfma_m<16>(x, codes, scales, y, N, K, p, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q4w
