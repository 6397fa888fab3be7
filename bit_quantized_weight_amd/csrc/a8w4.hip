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
//  * Activations are quantized into the workspace in the MFMA operand order,
//    so a wave copies each 32 x 32 operand (1 KB) from the workspace straight
//    into LDS with one buffer load that writes LDS; weight codes are unpacked
//    into LDS with an XOR swizzle (conflict-free 128-bit reads), and each
//    column's two block scales sit in one 8-byte entry (the magic offset term
//    is formed from them when they are read).

#include "q4w_internal.h"
#include <hip/hip_fp16.h>
#include <algorithm>
#include <cstddef>

namespace q4w {
namespace {

constexpr int kA8CounterWords = 512;   // arrival counters of the chunk-balanced GEMM

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

// quant127 with the division replaced by a product with rs = v_rcp_f32(sa)
// (1 ulp), rs = 0 when sa == 0.  Since |x / sa| <= 127.01, y = x rs is within
// 2^-15 of the correctly rounded quotient v = fl(x / sa), so
// round_half_away(y) = sign(y) floor(|y| + 1/2) equals round_half_away(v)
// unless |y| + 1/2 lies within 2^-12 of an integer; there (about 0.05% of
// elements) the correctly rounded division decides.
__device__ __forceinline__ int quant127_rcp(float x, float sa, float rs) {
  const float y = x * rs;
  const float t = fabsf(y) + 0.5f;
  const float fl = floorf(t);
  const float f = t - fl;
  if (fminf(f, 1.0f - f) < 0x1p-12f) return quant127(x, sa);
  const float q = fminf(copysignf(fl, y), 127.0f);
  return (int)fmaxf(q, -127.0f);
}

__device__ __forceinline__ float rcp_or_zero(float sa) {
  return sa == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sa);
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
  const float rs = rcp_or_zero(s);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= ((uint32_t)quant127_rcp(v[i], s, rs) & 0xFFu) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= ((uint32_t)quant127_rcp(v[4 + i], s, rs) & 0xFFu) << (8 * i);
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
                                                             float* __restrict__ sa_t,
                                                             uint32_t* __restrict__ counters) {
  // the GEMM's arrival counters start at zero (each GEMM leaves them so)
  if (counters && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < kA8CounterWords; i += 64) counters[i] = 0;
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
  const float rs = rcp_or_zero(s);
  constexpr int perm[16] = {0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15};
#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    uint32_t wv[4] = {0, 0, 0, 0};
#pragma unroll
    for (int sidx = 0; sidx < 16; ++sidx)
      wv[sidx >> 2] |= ((uint32_t)quant127_rcp(v[bi][perm[sidx]], s, rs) & 0xFFu) << (8 * (sidx & 3));
    const int b = 2 * g + bi;
    xq_t[((size_t)mt * nb + b) * 64 + l] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  if (h == 0) sa_t[((size_t)mt * G + g) * 32 + r] = s;
}

// ---- int8 MFMA GEMM --------------------------------------------------------
// The fp32 rescale (1.5 FMAs per output element and 32-wide block, the
// three-FMA magic-number form) costs three times the MFMA issue time, so the
// kernel is VALU-bound.  Everything else is kept off the VALU where it can
// be: the nibble -> int8 unpack and the weight-scale preparation are done
// once per workgroup into LDS, the activation tile is copied from the
// workspace straight into LDS by buffer loads with the LDS destination (no
// registers, no VALU), and the matrix-core products are software-pipelined
// one 32 x 32 subtile ahead of their rescale, so a wave issues the next
// pair of MFMAs and then rescales the previous pair while they run.  Every
// operand is staged in LDS one chunk ahead (double buffer), and two
// workgroups fit on a CU.
constexpr int kTM = 128;          // workgroup tile rows (tokens)
constexpr int kTN = 128;          // workgroup tile columns (output features)
constexpr int kChunkBlocks = 4;   // weight blocks per LDS chunk (128 K)
constexpr int kChunkGroups = kChunkBlocks / 2;
constexpr int kMSub = kTM / 32;   // 32-row MFMA subtiles per workgroup
constexpr int kNSub = kTN / 32;   // 32-column MFMA subtiles per workgroup
constexpr float kMagic = 12582912.0f;   // 0x4B400000 = 1.5 * 2^23
constexpr int kA8NarrowTiles = 256;      // fewer 128-row tiles than CUs: use 64-row tiles

__device__ __forceinline__ uint32_t lo_codes(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t hi_codes(uint32_t w) { return w & 0xF0F0F0F0u; }

// One LDS chunk buffer (35 KB).
//   bq: int8 B operands (16 x the codes), [n-subtile][block][slot], 16 B per
//       slot; the operand of MFMA lane l for block b sits in slot l ^ 4b, so
//       the staging writes (4 rows x 4 blocks per 16 lanes) and the operand
//       reads (16 consecutive lanes) both touch 16 distinct bank groups.
//   aq: int8 A operands, [m-subtile][block][lane], a straight copy of the
//       tiled activation layout.
//   dn: per group and column, {d[n, 2g] / 16, d[n, 2g+1] / 16}: one 8-byte
//       read gives a lane both block scales of its column.
//   sa: activation scales, [group][row].
struct ChunkLds {
  uint4 bq[kNSub * kChunkBlocks * 64];
  uint4 aq[kMSub * kChunkBlocks * 64];
  float2 dn[kChunkGroups * kTN];
  float sa[kChunkGroups * kTM];
};
// The raw codes of one chunk (128 rows x 4 blocks, 8 KB), copied from memory
// straight into LDS; unpacked into a chunk buffer's bq at the chunk's commit.
constexpr int kRawUnits = kTN * kChunkBlocks;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// kMS: 32-row M subtiles per workgroup, 4 (128 x 128 tiles) or 2 (64 x 128
// tiles, twice the workgroups for short prompts); each wave takes kMS / 2.
// kSplit: the chunk-balanced form, for tile counts a little above one round
// of the gridDim.x resident workgroups.  The tiles' K chunks, taken tile
// after tile, are cut into gridDim.x equal ranges of upw chunks, one per
// workgroup.  A tile cut by a range boundary is summed by the workgroups
// that share it: each writes its fp32 partial tile to the workspace, and the
// last to arrive adds the parts in range order (a fixed order: the result
// does not depend on which arrives last) and stores y.  With kDebug every
// chunk's block sums are written by the one workgroup that computes them.
template <bool kDebug, int kMS, bool kSplit>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(2, 2)))
a8w4_gemm_kernel(const uint4* __restrict__ xq_t, const float* __restrict__ sa_t,
                 const uint4* __restrict__ codes, const uint16_t* __restrict__ scales,
                 uint16_t* __restrict__ y, int32_t* __restrict__ acc_dbg, int M, int N, int K,
                 int mtiles, int ntiles, int upw, float* __restrict__ partial,
                 uint32_t* __restrict__ counters) {
  // The two chunk buffers are separate objects (not one array) so that the
  // compiler can tell the buffer being read from the one the next chunk's
  // loads are writing into; with one array it waits for those loads before
  // every LDS read.
  __shared__ ChunkLds lds0, lds1;
  __shared__ uint4 rawq[kRawUnits];
  __shared__ int is_last;
  static_assert(kMS == 2 || kMS == 4, "64- or 128-row tiles");
  constexpr int TM = 32 * kMS;      // rows (tokens) of this workgroup's tile
  constexpr int kMI = kMS / 2;      // 32-row subtiles per wave
  constexpr int kUPG = 2 * kMI;     // 32 x 32 subtiles (units) of a wave per group
  constexpr int kUnits = kChunkGroups * kUPG;

  const int nb = K / kBlock;
  const int G = K / kActGroup;
  const int nchunks = (nb + kChunkBlocks - 1) / kChunkBlocks;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
  const int lane = tid & 63;
  const int wm = wave >> 1;          // 2 x 2 waves, each (32 kMI) x 64
  const int wn = wave & 1;
  const int j = lane & 31;
  const int h = lane >> 5;

  v16i magic;
#pragma unroll
  for (int v = 0; v < 16; ++v) magic[v] = 0x4B400000;
  float acc[kMI][2][16];

  // Per-lane LDS byte offsets inside a chunk buffer; every operand read below
  // is one of these plus a compile-time offset.
  const int off_a = (int)offsetof(ChunkLds, aq) + ((wm * kMI * kChunkBlocks) * 64 + lane) * 16;
  int off_b[kChunkBlocks];
#pragma unroll
  for (int bl = 0; bl < kChunkBlocks; ++bl)
    off_b[bl] = (int)offsetof(ChunkLds, bq) + ((wn * 2 * kChunkBlocks) * 64 + (lane ^ (4 * bl))) * 16;
  const int off_dn = (int)offsetof(ChunkLds, dn) + (wn * 64 + j) * 8;
  const int off_sa = (int)offsetof(ChunkLds, sa) + (wm * 32 * kMI + 4 * h) * 4;

  // ---- chunks [c0, c1) of tile t into acc ---------------------------------
  // Tiles are numbered column-major (t = nt * mtiles + mt): neighbouring
  // tiles share their weight columns.
  auto segment = [&](int t, int c0, int c1) {
    const int mt = t % mtiles;
    const int nt = t / mtiles;
    const int n_base = nt * kTN;
    const int mt32 = mt * kMS;       // first 32-row activation tile of the workgroup

    // ---- buffer resources (out-of-range offsets read zeros, no traffic) ----
    const int rows_here = min(kTN, N - n_base);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(codes + (size_t)n_base * nb), 0, rows_here * nb * kBlockBytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(xq_t + (size_t)mt32 * nb * 64), 0, kMS * nb * 64 * 16, 0x00020000);

    // ---- cooperative chunk staging ------------------------------------------
    // The weight codes (2 units (row, block) of 16 B per thread) and the
    // activation tile (kMS units per thread) go straight to LDS; unless
    // kDebug, one pair of block scales (row, group) and one activation scale
    // per thread go through registers.  The
    // per-lane offsets are fixed for the segment; a chunk adds uniform steps.
    // In a chunk past the last block (K % 128 == 64) the code loads of blocks
    // nb, nb + 1 read the next row's first blocks (the buffer range check
    // gives zeros past the last row) and the activation loads the next
    // subtile's: finite values whose group is multiplied by d = 0, because
    // the scale loads, like the activation-scale loads, read zeros past the
    // last block (a wave-uniform test gives them an empty buffer resource).
    uint32_t rawd;
    float rawsa;
    const uint32_t ob = (uint32_t)(((tid >> 2) * nb + (tid & 3)) * kBlockBytes);   // unit it: + it * 64 rows
    const uint32_t ob_rows = (uint32_t)(64 * nb * kBlockBytes);
    const uint32_t oa = (uint32_t)((wave * 64 + lane) * 16);
    const int sgi = wave >> 1;                                 // scale pair: group of the chunk (tid >> 7)
    const uint32_t od = (uint32_t)(((tid & 127) * nb + 2 * sgi) * 2);
    const int agi = (wave * 64) / TM;                          // activation scale: group of the chunk (tid / TM)
    const uint32_t osa = (uint32_t)((((tid % TM) >> 5) * G * 32 + (tid & 31)) * 4);
    auto stage_issue = [&](int c, ChunkLds& L) {
  #pragma unroll
      for (int it = 0; it < 2; ++it)    // unit it * 256 + tid of rawq: row tid / 4 + 64 it, block tid % 4
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rc, (lds_ptr_t)(&rawq[it * 256 + wave * 64]), 16, ob + it * ob_rows + c * kChunkBlocks * kBlockBytes,
            0, 0, 0);
      // activation operands: wave w copies, for every m-subtile it, the
      // 1 KB of block c * 4 + w (64 lanes x 16 B) to aq[it][w][lane]
  #pragma unroll
      for (int it = 0; it < kMS; ++it)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (lds_ptr_t)(&L.aq[(it * kChunkBlocks + wave) * 64]), 16, oa,
            (it * nb + c * kChunkBlocks) * 64 * 16, 0, 0);
      if (!kDebug) {
        const bool dlive = c * kChunkBlocks + 2 * sgi < nb;     // wave-uniform
        const __amdgpu_buffer_rsrc_t rsd = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(scales + (size_t)n_base * nb), 0, dlive ? rows_here * nb * 2 : 0, 0x00020000);
        rawd = __builtin_amdgcn_raw_buffer_load_b32(rsd, od, c * kChunkBlocks * 2, 0);
        const int g = c * kChunkGroups + agi;
        const bool alive = agi < kChunkGroups && g < G;        // wave-uniform
        const __amdgpu_buffer_rsrc_t rsl = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(sa_t + (size_t)mt32 * G * 32), 0, alive ? kMS * G * 32 * 4 : 0, 0x00020000);
        rawsa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsl, osa, g * 32 * 4, 0));
      }
    };
    // Waits for the chunk's loads (the raw codes a thread unpacks are the
    // ones its own lane copied into LDS).
    auto stage_commit = [&](ChunkLds& L) {
      __builtin_amdgcn_s_waitcnt(0);
      // keep the scale conversions here, not next to the loads (they would
      // wait for them at the start of the chunk)
      if (!kDebug) asm volatile("" : "+v"(rawd), "+v"(rawsa));
  #pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int u = it * 256 + tid;
        const int r = u >> 2, bl = u & 3;
        const int ns = r >> 5, jj = r & 31;
        const uint4 w = rawq[u];
        // K-half 0 of the block is code words 0-1, half 1 is words 2-3
        L.bq[(ns * kChunkBlocks + bl) * 64 + (jj ^ (4 * bl))] =
            make_uint4(lo_codes(w.x), hi_codes(w.x), lo_codes(w.y), hi_codes(w.y));
        L.bq[(ns * kChunkBlocks + bl) * 64 + ((jj + 32) ^ (4 * bl))] =
            make_uint4(lo_codes(w.z), hi_codes(w.z), lo_codes(w.w), hi_codes(w.w));
      }
      if (!kDebug) {
        // the B operand carries 16 q: fold the 1/16 into the scales (exact).
        // Past the last block the loads read zeros: d = 0, so the group adds 0.
        const float d0 = __half2float(__ushort_as_half((unsigned short)(rawd & 0xFFFFu))) * 0.0625f;
        const float d1 = __half2float(__ushort_as_half((unsigned short)(rawd >> 16))) * 0.0625f;
        L.dn[tid] = make_float2(d0, d1);
        if (tid < kChunkGroups * TM) L.sa[tid] = rawsa;
      }
    };

#pragma unroll
    for (int a = 0; a < kMI; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    stage_issue(c0, lds0);
    stage_commit(lds0);
    __builtin_amdgcn_s_waitcnt(0);      // the activation tile has landed in LDS
    __syncthreads();

    // chunk c: computed from cur while chunk c + 1 is loaded into nxt
    auto chunk = [&](int c, const ChunkLds& cur, ChunkLds& nxt) {
      const char* L = reinterpret_cast<const char*>(&cur);
      if (c + 1 < c1) stage_issue(c + 1, nxt);

      // Unit u = (group gi, m-subtile mi, n-subtile ni) is one 32 x 32
      // subtile of one group: two MFMAs (the group's two blocks), then 16
      // values x 3 FMAs of rescale.  The MFMAs of unit u + 1 are issued
      // before the rescale of unit u.
      v4i av[kMI][2], bv[2][2];
      float4 dnv[2];      // per n-subtile: d0 / 16, d1 / 16, -1.5 * 2^23 * (d0 + d1) / 16
      float sav[16];
      auto load_group = [&](int gi) {
  #pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
  #pragma unroll
          for (int bi = 0; bi < 2; ++bi) {
            const uint4 t = *reinterpret_cast<const uint4*>(
                L + off_a + ((mi * kChunkBlocks + 2 * gi + bi) * 64) * 16);
            av[mi][bi] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
          }
  #pragma unroll
        for (int ni = 0; ni < 2; ++ni)
  #pragma unroll
          for (int bi = 0; bi < 2; ++bi) {
            const uint4 t = *reinterpret_cast<const uint4*>(
                L + off_b[2 * gi + bi] + ((ni * kChunkBlocks + 2 * gi + bi) * 64) * 16);
            bv[ni][bi] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
          }
      };
      auto load_dn = [&](int gi) {
        if (!kDebug) {
  #pragma unroll
          for (int ni = 0; ni < 2; ++ni)
          {
            const float2 t = *reinterpret_cast<const float2*>(L + off_dn + (gi * kTN + ni * 32) * 8);
            dnv[ni] = make_float4(t.x, t.y, -kMagic * (t.x + t.y), 0.f);
          }
        }
      };
      auto load_sa = [&](int gi, int mi, float (&s)[16]) {
        if (!kDebug) {
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float4 f = *reinterpret_cast<const float4*>(L + off_sa + (gi * TM + mi * 32 + 8 * r) * 4);
            s[4 * r + 0] = f.x; s[4 * r + 1] = f.y; s[4 * r + 2] = f.z; s[4 * r + 3] = f.w;
          }
        }
      };

      // The order below is pinned with empty asm statements that "modify"
      // the MFMA inputs just before each issue and each unit's accumulators
      // just after its rescale; without them the compiler hoists every MFMA
      // of the chunk to the top, and their results no longer fit in registers.
      // mfma_pair issues a unit's two MFMAs into d0, d1; the asm after them
      // also "touches" c0, c1 (the previous unit's results), so that unit's
      // rescale cannot start before this issue.
      auto mfma_pair = [&](int mi, int ni, v16i& d0, v16i& d1, v16i& c0, v16i& c1) {
        asm volatile("" : "+v"(av[mi][0]), "+v"(av[mi][1]), "+v"(bv[ni][0]), "+v"(bv[ni][1]));
        d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mi][0], bv[ni][0], magic, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mi][1], bv[ni][1], magic, 0, 0, 0);
        asm volatile("" : "+v"(d0), "+v"(d1), "+v"(c0), "+v"(c1));
      };
      v16i dc0, dc1;      // the unit being rescaled
      load_group(0);
      load_dn(0);
      load_sa(0, 0, sav);
      asm volatile("" : "+v"(av[0][0]), "+v"(av[0][1]), "+v"(bv[0][0]), "+v"(bv[0][1]));
      dc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[0][0], bv[0][0], magic, 0, 0, 0);
      dc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[0][1], bv[0][1], magic, 0, 0, 0);
      asm volatile("" : "+v"(dc0), "+v"(dc1));
  #pragma unroll
      for (int u = 0; u < kUnits; ++u) {
        const int gi = u / kUPG, mi = (u >> 1) % kMI, ni = u & 1;
        v16i dn0, dn1;
        if (u + 1 < kUnits) {
          const int u1 = u + 1;
          const int gi1 = u1 / kUPG, mi1 = (u1 >> 1) % kMI, ni1 = u1 & 1;
          if (u1 % kUPG == 0) load_group(gi1);
          mfma_pair(mi1, ni1, dn0, dn1, dc0, dc1);
        }
        const int g = c * kChunkGroups + gi;
        if (kDebug) {
          const int ncol = n_base + (wn * 2 + ni) * 32 + j;
  #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int mrow = (mt32 + wm * kMI + mi) * kA8TileM + 8 * (v >> 2) + 4 * h + (v & 3);
            if (mrow < M && ncol < N && g < G) {
              int32_t* o = acc_dbg + ((size_t)mrow * N + ncol) * nb + 2 * g;
              o[0] = (dc0[v] - 0x4B400000) >> 4;
              o[1] = (dc1[v] - 0x4B400000) >> 4;
            }
          }
        } else {
          const float4 d = dnv[ni];
          const float* sv = sav;
  #pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float s = fmaf(__int_as_float(dc0[v]), d.x, fmaf(__int_as_float(dc1[v]), d.y, d.z));
            acc[mi][ni][v] = fmaf(s, sv[v], acc[mi][ni][v]);
          }
  #pragma unroll
          for (int v = 0; v < 16; v += 4)
            asm volatile("" : "+v"(acc[mi][ni][v]), "+v"(acc[mi][ni][v + 1]), "+v"(acc[mi][ni][v + 2]),
                         "+v"(acc[mi][ni][v + 3]));
        }
        if (u + 1 < kUnits) {
          dc0 = dn0;
          dc1 = dn1;
          // the scales of the next unit, when they change (read here rather
          // than one unit ahead: one set of registers)
          const int u1 = u + 1;
          if (u1 % kUPG == 0) load_dn(u1 / kUPG);
          if ((u1 & 1) == 0) load_sa(u1 / kUPG, (u1 >> 1) % kMI, sav);
        }
        // keep the scheduler from hoisting later units' MFMAs (each holds
        // 32 result registers) above this unit's rescale
        __builtin_amdgcn_sched_barrier(0);
      }
      stage_commit(nxt);                         // past the segment: never read
      __builtin_amdgcn_s_waitcnt(0);             // the next activation tile has landed
      __syncthreads();
    };
#pragma unroll 1
    for (int c = c0; c < c1; c += 2) {
      chunk(c, lds0, lds1);
      if (c + 1 < c1) chunk(c + 1, lds1, lds0);
    }
  };

  // ---- y of tile t -----------------------------------------------------------
  // The value of output (mi, ni, v) is produced by get(mi, ni, v).
  auto store_y = [&](int t, auto get) {
    const int n_base = (t / mtiles) * kTN;
    const int mt32 = (t % mtiles) * kMS;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int ncol = n_base + (wn * 2 + ni) * 32 + j;
        float r[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) r[v] = get(mi, ni, v);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int mrow = (mt32 + wm * kMI + mi) * kA8TileM + 8 * (v >> 2) + 4 * h + (v & 3);
          if (mrow < M && ncol < N) y[(size_t)mrow * N + ncol] = __half_as_ushort(__float2half_rn(r[v]));
        }
      }
  };
  auto own = [&](int mi, int ni, int v) { return acc[mi][ni][v]; };

  if constexpr (!kSplit) {
    // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs,
    // so give each XCD its own tiles, which then share its L2.  With whole
    // weight columns per XCD and at least 16 token tiles, an XCD walks its
    // columns in two halves of the token tiles: its 64 resident workgroups
    // then cover 8 columns x 8 token tiles (a smaller working set per K
    // chunk than 4 columns x 16 token tiles; measured at M = 2048, N = 17408:
    // L2 misses -39%, 0.380 -> 0.375 ms).  Otherwise a contiguous range of
    // tiles per XCD.
    const int total = mtiles * ntiles;
    int bid = blockIdx.x;
    if ((ntiles & 7) == 0 && mtiles >= 16 && (mtiles & 1) == 0) {
      const int x = bid & 7, i = bid >> 3;
      const int cols = ntiles >> 3, gm = mtiles >> 1;
      const int half = i / (cols * gm), rem = i - half * cols * gm;
      bid = (x * cols + rem / gm) * mtiles + half * gm + rem % gm;
    } else if ((total & 7) == 0) {
      bid = (bid & 7) * (total >> 3) + (bid >> 3);
    }
    segment(bid, 0, nchunks);
    if (!kDebug) store_y(bid, own);
  } else {
    // contiguous ranges per XCD, as above (the grid is a multiple of 8)
    const int i = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
    const int W = mtiles * ntiles * nchunks;
    const int u1 = min(W, (i + 1) * upw);
    for (int u = i * upw; u < u1;) {
      const int t = u / nchunks;
      const int c0 = u - t * nchunks;
      const int c1 = min(nchunks, c0 + (u1 - u));
      segment(t, c0, c1);
      u += c1 - c0;
      if (kDebug) continue;          // block sums were written by segment()
      if (c0 == 0 && c1 == nchunks) {
        store_y(t, own);
        continue;
      }
      // Tile t is shared by workgroups ia..ib.  Workgroup w keeps its part
      // in slot 2w when the part is the first of w's range, else 2w + 1
      // (a range has at most one part that starts and one that ends inside
      // a tile).  64 floats per thread and slot, thread-minor.
      const int tu = t * nchunks;               // first unit of tile t
      const int ia = tu / upw;
      const int ib = (tu + nchunks - 1) / upw;
      auto slot = [&](int w) {
        return partial + (size_t)(w * upw >= tu ? 2 * w : 2 * w + 1) * (64 * 256) + tid;
      };
      float* mine = slot(i);
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            __hip_atomic_store(mine + ((mi * 2 + ni) * 16 + v) * 256, acc[mi][ni][v], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        is_last = __hip_atomic_fetch_add(&counters[ia], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (unsigned)(ib - ia);
      __syncthreads();
      if (is_last) {
        // the parts in range order, whichever workgroup arrived last
        store_y(t, [&](int mi, int ni, int v) {
          float r = 0.f;
          for (int w = ia; w <= ib; ++w)
            r += w == i ? acc[mi][ni][v]
                        : __hip_atomic_load(slot(w) + ((mi * 2 + ni) * 16 + v) * 256, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
          return r;
        });
        if (tid == 0) __hip_atomic_store(&counters[ia], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace

int64_t a8_padded_rows(int64_t M) { return ((M + kTM - 1) / kTM) * kTM; }

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Chunk-balanced form: kA8Slots workgroups (two per CU) share the tiles'
// chunks.  Its region (arrival counters, then two fp32 partial tiles per
// workgroup) follows the activations in workspaces of at least
// kA8SplitMinRows padded rows.
constexpr int kA8Slots = kA8CounterWords;
constexpr int64_t kA8SplitMinRows = 256;
constexpr size_t kA8CounterBytes = kA8Slots * sizeof(uint32_t);
constexpr size_t kA8PartialBytes = (size_t)2 * kA8Slots * 64 * 256 * sizeof(float);

static size_t a8_act_bytes(int64_t mp, int64_t K) {
  return align256((size_t)mp * K) + align256((size_t)mp * (K / kActGroup) * sizeof(float));
}

size_t a8_ws_bytes(int64_t M, int64_t K) {
  const int64_t mp = a8_padded_rows(M);
  return a8_act_bytes(mp, K) + (mp >= kA8SplitMinRows ? align256(kA8CounterBytes) + kA8PartialBytes : 0);
}

hipError_t launch_act_quant_rowmajor(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* sa,
                                     hipStream_t s) {
  const int G = (int)(K / kActGroup);
  // Rows are independent: pieces of at most 2^25 groups (2^28 work-items,
  // 8 per group) keep a launch far below 2^32 work-items.
  const int64_t rows_per_piece = std::max<int64_t>(1, (int64_t(1) << 25) / G);
  for (int64_t m0 = 0; m0 < M; m0 += rows_per_piece) {
    const int64_t rows = std::min(rows_per_piece, M - m0);
    const int64_t ngroups = rows * G;
    const int64_t grid = (ngroups * 8 + 255) / 256;
    hipLaunchKernelGGL(act_quant_rowmajor_kernel, dim3((unsigned)grid), dim3(256), 0, s, x + m0 * K, ngroups,
                       G, (int)K, xq + m0 * K, sa + m0 * G);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_act_quant_tiled(const uint16_t* x, int64_t M, int64_t K, void* ws, hipStream_t s) {
  const int64_t mp = a8_padded_rows(M);
  uint4* xq_t = reinterpret_cast<uint4*>(ws);
  float* sa_t = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)mp * K));
  uint32_t* counters = mp >= kA8SplitMinRows
                           ? reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + a8_act_bytes(mp, K))
                           : nullptr;
  hipLaunchKernelGGL(act_quant_tiled_kernel, dim3((unsigned)(K / kActGroup), (unsigned)(mp / kA8TileM)),
                     dim3(64), 0, s, x, (int)M, (int)K, xq_t, sa_t, counters);
  return hipGetLastError();
}

hipError_t launch_a8w4_gemm(const void* ws, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                            int32_t* acc_debug, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  const int64_t mp = a8_padded_rows(M);
  const uint4* xq_t = reinterpret_cast<const uint4*>(ws);
  const float* sa_t = reinterpret_cast<const float*>(static_cast<const char*>(ws) + align256((size_t)mp * K));
  const int ntiles = (int)((N + kTN - 1) / kTN);
  const int nchunks = (int)((K / kBlock + kChunkBlocks - 1) / kChunkBlocks);
  const int64_t tiles = (mp / kTM) * ntiles;
  // Chunk-balanced form when the 128 x 128 tiles make one round of the
  // resident slots and at most half another (a range then spans more than
  // one tile).  Measured per GEMM: at M = 2048 (640 tiles) down 550 -> 473 us
  // and out 163 -> 157 us; at M = 512 (544 tiles) gate 164 -> 145 us.  At
  // 896 tiles (qkv, M = 2048) it measured 6% slower, at 1088 no better and at
  // 2176 (gate, M = 2048) 10% slower, so larger counts run the plain form.
  const bool split = mp >= kA8SplitMinRows && tiles > kA8Slots &&
                     tiles <= kA8Slots + kA8Slots / 2 && tiles * nchunks < (int64_t)1 << 30;
  // 64-row tiles when 128-row tiles would leave CUs idle (measured at M = 512:
  // qkv 81 -> 71 us, out 75 -> 63, down 239 -> 205; at 320..448 tiles the
  // 128-row form stays faster)
  const bool narrow = !split && tiles < kA8NarrowTiles;
  const int mtiles = (int)(mp / (narrow ? kTM / 2 : kTM));
  int upw = 0;
  uint32_t* counters = nullptr;
  float* partial = nullptr;
  dim3 grid((unsigned)(mtiles * ntiles));
  if (split) {
    const int64_t units = tiles * nchunks;
    upw = (int)((units + kA8Slots - 1) / kA8Slots);
    grid = dim3(kA8Slots);
    char* region = static_cast<char*>(const_cast<void*>(ws)) + a8_act_bytes(mp, K);
    counters = reinterpret_cast<uint32_t*>(region);
    partial = reinterpret_cast<float*>(region + align256(kA8CounterBytes));
  }
#define Q4W_A8_LAUNCH(DBG, MS, SPLIT)                                                             \
  hipLaunchKernelGGL((a8w4_gemm_kernel<DBG, MS, SPLIT>), grid, dim3(256), 0, s, xq_t, sa_t,      \
                     reinterpret_cast<const uint4*>(codes), scales, y, acc_debug, (int)M, (int)N, \
                     (int)K, mtiles, ntiles, upw, partial, counters)
  if (acc_debug) {
    if (split) Q4W_A8_LAUNCH(true, 4, true);
    else if (narrow) Q4W_A8_LAUNCH(true, 2, false);
    else Q4W_A8_LAUNCH(true, 4, false);
  } else if (split) {
    Q4W_A8_LAUNCH(false, 4, true);
  } else {
    if (narrow) Q4W_A8_LAUNCH(false, 2, false);
    else Q4W_A8_LAUNCH(false, 4, false);
  }
#undef Q4W_A8_LAUNCH
  return hipGetLastError();
}

}  // namespace q4w
