// q4_gemv_skinny: Y[M, N] = X[M, K] . What^T for small M -- the weight stream
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
//  * A wave is 2 row-slots x 32 lanes.  Lane j of a slot owns 32-weight blocks
//    j, j+32, j+64, ... of its rows, so one 128-bit load of a wave reads two
//    rows x 512 contiguous bytes of codes.  Each lane carries RL rows and
//    re-uses its activation registers RL times.
//  * Every step of a workgroup's K-slice is requested up front (a register
//    ring when the slice is longer than the ring): on MI355X a 50 MB stream
//    only reaches full bandwidth when each wave has all of its bytes in
//    flight at once.  Lanes past the end of the slice use an out-of-range
//    buffer offset, which returns zeros without touching memory.
//  * Activations are staged once per workgroup into LDS in a permuted fp16
//    layout matching the in-register unpack below, plus a per-block bias.
//    Their loads are issued before the weight loads: loads complete in issue
//    order, and behind the weight stream of every other wave they would
//    otherwise hold up the start of the compute.
//  * Unpack: (w & 0x000F000F) ^ 0x64086408 flips each nibble's sign bit
//    (two's complement q -> u = q + 8) and inserts the fp16 exponent of 1024
//    (mantissa LSB = 1), giving the pair (1024 + u0, 1024 + u4) in one
//    v_bitop3.  Odd nibbles sit 4 bits higher, so they get the exponent of 64
//    (mantissa LSB = 1/16): (w & 0x00F000F0) ^ 0x54805480 = (64 + u1, 64 + u5).
//    v_dot2_f32_f16 accumulates in fp32 against unscaled fp16 activations and
//    the constant parts (1032 per even, 72 per odd activation) are removed
//    exactly by starting each block's accumulator at -bias.  The block scale
//    multiplies the block partial once (fp32 FMA).
//  * 32-lane DPP/swizzle reduction per row.  K can be split over workgroups
//    (split-K) whose fp32 partials are summed in a fixed order by the last
//    workgroup to arrive (one kernel, deterministic, no cache flushes).

#include "q4w_internal.h"
#include "splitk.h"
#include <hip/hip_fp16.h>

namespace q4w {
namespace {

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kFixupBatch = 16;         // split-K fixup: partial loads in flight per thread
constexpr int kLanesPerRow = 32;        // lanes sharing one row along K
constexpr int kSlots = 64 / kLanesPerRow;
constexpr int kLdsBudget = 48 * 1024;   // activation staging bytes per workgroup
constexpr int kMinSkinnyWgs = 256;      // one workgroup per CU
constexpr int kCachePolicyNT = 2;       // buffer-load cache policy bit: non-temporal (streaming)
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any resource

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Word 3 of a gfx9 buffer resource: 32-bit data format, raw (untyped) access.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// Sum over each 32-lane half of the wave; every lane of the half gets the total.
__device__ __forceinline__ float half_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));  // row_ror:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));  // row_ror:1
  // lane l and lane l ^ 16 (bitmask swizzle: and 0x1F, xor 0x10)
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return v;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace

// Rows per lane: more rows re-use the activation registers more (less LDS
// traffic per weight) at the cost of registers and of fewer workgroups.
// (This kernel serves M = 1..3; wider M goes to the matrix-core kernels.)
__host__ __device__ constexpr int rows_per_lane(int) { return 2; }
// Steps requested at once per wave (the register ring).
__host__ __device__ constexpr int ring_steps(int M) { return M <= 2 ? 6 : 5; }
// Longest slice when a row must be split: above M = 1 more workgroups pay off
// (verify_down M = 2: 5 slices of 4 steps 14.2 us, 3 slices of 6 steps 15.2 us).
__host__ __device__ constexpr int split_steps(int M) { return M == 1 ? 6 : 4; }
constexpr int kShortSlice = 4;           // depth of the short no-refill form
// Occupancy target (waves per SIMD).
__host__ __device__ constexpr int waves_per_simd(int) { return 4; }
// Largest slice (blocks): whole steps, within the LDS budget and at most two
// rings long (one from M = 3 on); and the (row, block) staging items per
// thread it needs.
__host__ __device__ constexpr int max_ring_rounds(int M) { return M >= 3 ? 1 : 2; }   // the refilled form would spill
__host__ __device__ constexpr int max_slice_blocks(int M) {
  return (kLdsBudget / (M * (4 * 16 + 4)) / kLanesPerRow) * kLanesPerRow <
                 max_ring_rounds(M) * ring_steps(M) * kLanesPerRow
             ? (kLdsBudget / (M * (4 * 16 + 4)) / kLanesPerRow) * kLanesPerRow
             : max_ring_rounds(M) * ring_steps(M) * kLanesPerRow;
}
__host__ __device__ constexpr int stage_items(int M) {
  return (M * max_slice_blocks(M) + kThreads - 1) / kThreads;
}

namespace {

// kRing = false: every slice fits the ring (steps <= P), one pass, no refills.
// P: steps of loads in flight per wave (the register ring).  The no-refill
// form is built at two depths: a slice of at most kShortSlice steps takes the
// short one (fewer registers, more waves per SIMD).
template <int M, bool kRing, int P>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(waves_per_simd(M), 8)))
skinny_kernel(const uint16_t* __restrict__ x, const uint4* __restrict__ codes,
              const uint16_t* __restrict__ scales, uint16_t* __restrict__ y,
              float* __restrict__ partial, uint32_t* __restrict__ counters,
              int N, int K, int bps, int S) {
  constexpr int RL = rows_per_lane(M);
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

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int slot = lane / kLanesPerRow;
  const int j = lane % kLanesPerRow;
  const int tile_row0 = tile * kRowsPerWg;
  const int rl0 = (wave * kSlots + slot) * RL;   // first row of this lane, tile-local

  // Buffer resources cover this workgroup's rows only; a lane whose row is
  // past N reads zeros (hardware range check), so rows need no clamping.
  const int rows_here = min(kRowsPerWg, N - tile_row0);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + (size_t)tile_row0 * nb), 0, rows_here * nb * kBlockBytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + (size_t)tile_row0 * nb), 0, rows_here * nb * 2, kRsrcWord3);
  uint32_t vblk[RL];   // block index (tile-local) of this lane's block in step 0, per row
#pragma unroll
  for (int i = 0; i < RL; ++i) vblk[i] = (uint32_t)((rl0 + i) * nb + kb0 + j);

  // The ring: buf[p] holds step t with t % P == p.  A lane whose block is past
  // the slice end (including whole steps past the end) gets an out-of-range
  // offset: the load returns zeros without a memory request.
  uint4 buf[P][RL];
  uint32_t sbuf[P][RL];
  auto load_step = [&](int t, uint4 (&c)[RL], uint32_t (&sc)[RL]) {
    const bool live = t * kLanesPerRow + j < nbs;
#pragma unroll
    for (int i = 0; i < RL; ++i) {
      const uint32_t vo = live ? vblk[i] * kBlockBytes : kOutOfRange;
      const uint32_t so = live ? vblk[i] * 2 : kOutOfRange;
      // Non-temporal: every code byte is read once, as whole 128-byte lines
      // (a wave reads 2 rows x 512 B), so nothing is gained by keeping it in
      // the caches.  (The scales are read in half lines, which the next step
      // completes from L2, so they keep the default policy.)
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, t * kLanesPerRow * kBlockBytes, kCachePolicyNT);
      c[i] = make_uint4(v[0], v[1], v[2], v[3]);
      sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, t * kLanesPerRow * 2, 0);
    }
  };
  // ---- activation loads first: items (row m, block b) of this slice -----
  // They are needed before any weight step, and loads complete in issue
  // order, so they go out ahead of the weight loads.  Blocks past the slice
  // read zeros (out-of-range offset, no memory request).
  // (row, block) staging items per thread: a no-refill slice is at most P
  // steps.  At least two: with one, the compiler issues these loads after
  // the weight loads (measured: +0.4 to +0.9 us at M = 1).
  constexpr int kItems = kRing ? stage_items(M)
                               : ((M * P * kLanesPerRow + kThreads - 1) / kThreads > 2
                                      ? (M * P * kLanesPerRow + kThreads - 1) / kThreads : 2);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, M * K * 2, kRsrcWord3);
  uint4 raw[kItems][4];
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int u = tid + it * kThreads;
    const int m = u / bpad;
    const int b = u - m * bpad;
    const bool valid = u < M * bpad && b < nbs;
    const uint32_t xo = valid ? (uint32_t)(m * K + (kb0 + b) * kBlock) * 2 : kOutOfRange;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, q * 16, 0);
      raw[it][q] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }

#pragma unroll
  for (int p = 0; p < P; ++p) load_step(p, buf[p], sbuf[p]);

  uint4* xs = smem;                                          // [M][4][bpad] fp16 quads
  float* cs = reinterpret_cast<float*>(smem + M * 4 * bpad); // [M][bpad] -bias

  // ---- stage the activation slice in the unpack's pair order --------------
  const uint32_t k1032 = 0x64086408u;   // fp16 pair (1032, 1032)
  const uint32_t k72 = 0x54805480u;     // fp16 pair (72, 72)
#pragma unroll
  for (int it = 0; it < kItems; ++it) {
    const int u = tid + it * kThreads;
    if (u < M * bpad) {
      const int m = u / bpad;
      const int b = u - m * bpad;
      float c = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // raw holds elements e0..e7 of code word q as (e1:e0, e3:e2, e5:e4, e7:e6)
        const uint32_t w0 = raw[it][q].x, w1 = raw[it][q].y, w2 = raw[it][q].z, w3 = raw[it][q].w;
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
  }
  __syncthreads();

  // ---- stream the weights -----------------------------------------------
  float yacc[RL][M];
#pragma unroll
  for (int i = 0; i < RL; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) yacc[i][m] = 0.f;

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

  if (!kRing) {
    // the whole slice (steps <= P) is already in flight: no refills
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (p < steps) compute_step(p, buf[p], sbuf[p]);
  } else {
    // Refills are unconditional (past the end they are out-of-range, i.e.
    // no memory request): a conditional load makes the compiler wait for
    // every outstanding load at the merge point and serializes the ring.
#pragma unroll 1
    for (int t0 = 0; t0 < steps; t0 += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (t0 + p < steps) compute_step(t0 + p, buf[p], sbuf[p]);
        load_step(t0 + p + P, buf[p], sbuf[p]);
      }
    }
  }

  // ---- reduce the 32 lanes of each row; lane j then stores value j -------
  constexpr int kVals = RL * M;          // (row i, token m) pairs, index i * M + m
  static_assert(kVals <= kLanesPerRow, "one store pass");
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < RL; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float s = half_sum(yacc[i][m]);
      if (j == i * M + m) v = s;
    }
  if (j < kVals) {
    const int i = j / M;
    const int m = j - i * M;
    const int n = tile_row0 + rl0 + i;
    if (n < N) {
      if (S == 1) y[(size_t)m * N + n] = __half_as_ushort(__float2half_rn(v));
      else  // agent-coherent store: visible to every XCD once complete
        __hip_atomic_store(&partial[((size_t)split * M + m) * N + n], v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  if (S == 1) return;

  // ---- split-K: the last workgroup of this row tile sums the partials ----
  // Partials are written and read with agent-scope (cache-coherent) accesses,
  // so no L2 write-back or invalidate is needed: waiting for this
  // workgroup's stores to complete before the arrival count is enough.
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
  if (tid == 0)   // leave the workspace ready for the next call
    __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  const int steps = bpad / kLanesPerRow;
  const bool ring = steps > ring_steps(M);   // never when a slice is one ring at most
  if constexpr (max_ring_rounds(M) > 1) {
    if (ring) {
      hipLaunchKernelGGL((skinny_kernel<M, true, ring_steps(M)>), dim3(p.row_tiles, p.splits), dim3(kThreads), lds,
                         s, x, reinterpret_cast<const uint4*>(codes), scales, y, partial, counters,
                         (int)N, (int)K, p.blocks_per_split, p.splits);
      return hipGetLastError();
    }
  } else if (ring) {
    return hipErrorInvalidValue;
  }
  if (steps <= kShortSlice)
    hipLaunchKernelGGL((skinny_kernel<M, false, kShortSlice>), dim3(p.row_tiles, p.splits), dim3(kThreads),
                       lds, s, x, reinterpret_cast<const uint4*>(codes), scales, y, partial, counters,
                       (int)N, (int)K, p.blocks_per_split, p.splits);
  else
    hipLaunchKernelGGL((skinny_kernel<M, false, ring_steps(M)>), dim3(p.row_tiles, p.splits), dim3(kThreads),
                       lds, s, x, reinterpret_cast<const uint4*>(codes), scales, y, partial, counters,
                       (int)N, (int)K, p.blocks_per_split, p.splits);
  return hipGetLastError();
}

}  // namespace

// Split plan.  A slice is a whole number of 32-block steps and its
// activations fit the LDS budget (at most two rings long); S is as small as
// the rules below allow.  split_k > 0 asks for that many slices (raised when
// the LDS budget needs more).
SkinnyPlan plan_skinny(int M, int64_t N, int64_t K, int split_k) {
  if (M >= kMfmaMinM) return plan_skinny_mfma(M, N, K, split_k);
  if (M >= kMfma4MinM) return plan_skinny_mfma4(M, N, K, split_k);
  // At M = 3 the 4x4x4 kernel's short split slices beat this kernel's on
  // rows that need splitting (K = 17408, N = 5120: 15.31 -> 14.58 us); on
  // one-slice rows this kernel stays ahead (K = 5120, N = 7168: 7.42 against
  // 7.67 us), and at M = 2 it does on both (13.74 against 13.98 us).
  if (M == kMfma4SplitM && split_k <= 0 && K / kBlock > kMfma4SliceBlocks)
    return plan_skinny_mfma4(M, N, K, split_k);
  SkinnyPlan p{};
  p.route = kRouteDot2;
  p.rows_per_wg = kWaves * kSlots * rows_per_lane(M);
  p.row_tiles = (int)((N + p.rows_per_wg - 1) / p.rows_per_wg);
  const int nb = (int)(K / kBlock);
  const int lds_blocks = max_slice_blocks(M);                  // blocks of one slice in LDS
  int bps;
  if (split_k > 0) {
    bps = (nb + split_k - 1) / split_k;
    if (bps > lds_blocks) bps = lds_blocks;
  } else {
    // Split-K ends the launch with a chain of memory round trips (partial
    // stores, the arrival count, the last workgroup's partial loads).  On the
    // measured shapes that chain costs more than one ring refill, and more
    // than running with as few as one workgroup per CU, so: one slice when
    // the row fits the largest slice, else slices of split_steps(M) steps
    // (within one ring: no refill); more slices only below kMinSkinnyWgs
    // workgroups.
    const int steps_total = (nb + kLanesPerRow - 1) / kLanesPerRow;
    const int max_steps = lds_blocks / kLanesPerRow;            // largest slice
    const int sl = split_steps(M);
    int S = steps_total <= max_steps ? 1 : (steps_total + sl - 1) / sl;
    while ((int64_t)S * p.row_tiles < kMinSkinnyWgs && steps_total / (S + 1) >= 1) ++S;
    bps = ((steps_total + S - 1) / S) * kLanesPerRow;
  }
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
  if (p.route == kRouteMfma) return launch_skinny_mfma(x, codes, scales, y, M, N, K, p, ws, s);
  if (p.route == kRouteMfma4) return launch_skinny_mfma4(x, codes, scales, y, M, N, K, p, ws, s);
  switch (M) {
    case 1: return launch_m<1>(x, codes, scales, y, N, K, p, ws, s);
    case 2: return launch_m<2>(x, codes, scales, y, N, K, p, ws, s);
    case 3: return launch_m<3>(x, codes, scales, y, N, K, p, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill_zero_u16(uint16_t* y, int64_t count, hipStream_t s) {
  // pieces of at most 2^28 elements keep a launch far below 2^32 work-items
  constexpr int64_t kPiece = int64_t(1) << 28;
  for (int64_t c0 = 0; c0 < count; c0 += kPiece) {
    const int64_t n = count - c0 < kPiece ? count - c0 : kPiece;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y + c0, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace q4w
