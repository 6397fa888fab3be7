// q4_attn_decode: the decode-time attention read of a 4-bit K/V cache.
//
// Page 3 ("Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF"): 16 of the 64
// layers are full-attention layers whose K/V cache, held with 4-bit K and V,
// grows with the context (roughly 4.25 GiB at 256K), and those K/V reads are
// what takes decode from about 50 tok/s to 12.61 tok/s at a 261.5K-token
// cache.  For each of the M query tokens of a step (the last M cache
// positions: the target token and its drafts) and each query head h:
//   o[m, h] = sum_t softmax_t(q[m, h] . K[t, g] / sqrt(D)) V[t, g],  g = h / G,
// over the cache positions t <= T - M + m.  K and V are token-major rows of
// H_kv * D values in the weights' 32-element 4-bit block format.
//
// gfx950 design (bound by streaming the cache from HBM):
//  * One workgroup (8 waves) per (K/V head g, slice of the keys); a wave
//    takes 32-key tiles of its slice in turn and keeps its own running max,
//    sum and output (flash-decoding).  The R = M * G query rows of head g
//    are the columns of every matrix product, in RT tiles of 16 (RT = 1 up
//    to R = 16, i.e. up to three query tokens at G = 5; RT = 2 up to 32).
//  * All products are v_mfma_f32_16x16x32_f16; lane l has c = l % 16 and
//    slot group grp = l / 16.  Scores S^T[t, r]: A = K rows (key 16 h + c of
//    the tile's half h), B = Q^T (column r = 16 rt + c); D rows
//    4 grp .. 4 grp + 3.  Lane (c, grp) loads bytes [32 grp, 32 grp + 32) of
//    its key's 128 code bytes (blocks 2 grp and 2 grp + 1) and their two
//    scales, and dequantizes one code word per product into fp16
//    (magic-exponent nibble unpack, exact integer codes, one rounding of
//    q * d): product j takes channels 64 grp + 8 j .. + 7, and Q^T (in LDS)
//    holds the same channels in the unpack's pair order.
//  * Softmax in base 2, in fp32, with a lazy running max: the output is
//    rescaled (and the row max taken across the row's four lanes) only when
//    some score passes its row's max by more than 8 (p <= 256).
//  * Values: O^T[d, r] += V^T[d, t] P^T[t, r].  Slot 8 grp + 4 h + i of a
//    value product is key 16 h + 4 grp + i, so P^T, the B operand, is the
//    lane's own 8 probabilities.  The V codes are loaded 8 lanes per key row
//    (one 16-byte block each, so a load instruction covers 8 whole cache
//    lines) and dequantized into a wave-private LDS tile (512-byte rows); the
//    V^T operand comes out of it through two transposing reads per product
//    (ds_read_b64_tr_b16: keys 4 grp + 0..3 and 16 + 4 grp + 0..3 of one
//    channel).  16-byte chunk n of row t sits at n ^ f(t), f linear over the
//    bits of t % 8 (bit 0 -> 2, bit 1 -> 5, bit 2 -> 9), so that the row
//    writes (8 keys x 2 blocks per 16 lanes) and the transposing reads
//    (8 keys x 2 chunks per 32 lanes) meet no bank conflicts with 32 or 64
//    banks.
//  * A tile is read through buffer resources that start at the tile and end
//    at the cache's end (no bytes for a tile that does not exist), so each
//    lane's load offsets are fixed and keys past T read zeros.
//  * The 8 waves' partial results are combined in LDS, each workgroup writes
//    one partial (rows < R only), and a second kernel merges the slices.

#include "q4w_internal.h"
#include <hip/hip_fp16.h>

namespace q4w {
namespace {

constexpr int kD = kAttnHeadDim;          // head dimension (256)
constexpr int kTileKeys = 32;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kVRow = 512;                // bytes per dequantized V row in LDS
constexpr int kVTile = kTileKeys * kVRow; // bytes per wave's V tile
constexpr float kNegBig = -1.0e30f;       // running-max start (finite: no inf - inf)
constexpr float kRescaleGap = 8.0f;       // base-2 growth of the max that forces a rescale
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kMergeBatch = 16;           // slice loads in flight per thread in the merge

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// 8 codes of one 32-bit word (elements e0..e7) times the block scale, as
// fp16 pairs in the order (e0, e4), (e1, e5), (e2, e6), (e3, e7).
// (w & 0x000F000F) ^ 0x64086408 is the fp16 pair (1024 + u) with u = q + 8;
// odd nibbles sit 4 bits higher and take the exponent of 64 instead.
__device__ __forceinline__ uint4 dequant8(uint32_t w, h2 d2) {
  const uint32_t w8 = w >> 8;
  const h2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
  const h2 q0 = as_h2((w & 0x000F000Fu) ^ 0x64086408u) - c1032;    // exact codes
  const h2 q1 = as_h2((w & 0x00F000F0u) ^ 0x54805480u) - c72;
  const h2 q2 = as_h2((w8 & 0x000F000Fu) ^ 0x64086408u) - c1032;
  const h2 q3 = as_h2((w8 & 0x00F000F0u) ^ 0x54805480u) - c72;
  return make_uint4(as_u32(q0 * d2), as_u32(q1 * d2), as_u32(q2 * d2), as_u32(q3 * d2));
}

__device__ __forceinline__ h8 as_h8(uint4 v) { return __builtin_bit_cast(h8, v); }

// max of x over lanes l and l ^ 32
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---- kernel 1: one partial result per (K/V head, key slice) ---------------
// grid (S, H_kv), 8 waves.  Slice s covers the key tiles s + k S, k < tps:
// the slices interleave, so at any time all workgroups read neighbouring
// tiles (the whole chip sweeps the cache as one window, which streams faster
// than S separate regions).
// part_o: [S][H_kv][R][D] fp32, part_ml: [S][H_kv][R][2] (base-2 max, sum).

// f(t): the V tile's chunk swizzle of row t (linear over the bits of t % 8)
__device__ __forceinline__ int vt_swizzle(int t) {
  return (2 * (t & 1)) ^ (5 * ((t >> 1) & 1)) ^ (9 * ((t >> 2) & 1));
}

// max of x over lanes l and l ^ 16
__device__ __forceinline__ float rows16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int RT>
__global__ void __launch_bounds__(kThreads)
attn_partial_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_codes,
                    const uint16_t* __restrict__ k_scales, const uint8_t* __restrict__ v_codes,
                    const uint16_t* __restrict__ v_scales, float* __restrict__ part_o,
                    float* __restrict__ part_ml, int M, int Hq, int Hkv, int T, int tps) {
  static_assert(RT == 1 || RT == 2, "16 or 32 query rows");
  // LDS: Q^T B operands [rt][product j][lane] (uint4), then one dequantized V
  // tile per wave, [key][512 bytes].  After the key loop the whole area
  // serves the combine of the 8 waves.
  constexpr int kQtEntries = RT * 8 * 64;
  constexpr int kQtBytes = kQtEntries * 16;
  constexpr int kLdsBytes = kQtBytes + kWaves * kVTile;
  __shared__ __align__(16) unsigned char lds[kLdsBytes];
  uint4* qt = reinterpret_cast<uint4*>(lds);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 15;
  const int grp = lane >> 4;
  const int split = blockIdx.x;
  const int head = blockIdx.y;               // K/V head
  const int G = Hq / Hkv;
  const int R = M * G;
  const int ntiles = (T + kTileKeys - 1) / kTileKeys;
  const int S = gridDim.x;
  auto phys = [&](int k) { return k * S + split; };
  auto exists = [&](int k) { return k < tps && phys(k) < ntiles; };

  // ---- Q^T into LDS: entry (rt, j, lane') = Q[16 rt + c', 64 grp' + 8 j + (0,4,1,5,2,6,3,7)]
  for (int e = tid; e < kQtEntries; e += kThreads) {
    const int l2 = e & 63, j = (e >> 6) & 7, rt = e >> 9;
    const int r2 = 16 * rt + (l2 & 15), g2 = l2 >> 4;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (r2 < R) {
      const int m = r2 / G, hq = head * G + r2 % G;
      const uint4 w = *reinterpret_cast<const uint4*>(q + ((size_t)m * Hq + hq) * kD + 64 * g2 + 8 * j);
      o.x = (w.x & 0xFFFFu) | (w.z << 16);          // (e0, e4)
      o.y = (w.x >> 16) | (w.z & 0xFFFF0000u);      // (e1, e5)
      o.z = (w.y & 0xFFFFu) | (w.w << 16);          // (e2, e6)
      o.w = (w.y >> 16) | (w.w & 0xFFFF0000u);      // (e3, e7)
    }
    qt[e] = o;
  }
  __syncthreads();
  uint4 bq1[RT == 1 ? 8 : 1];                      // one row tile: Q^T held in registers
  if constexpr (RT == 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) bq1[j] = qt[j * 64 + lane];
  }

  const int row_codes = Hkv * kD / 2;
  const int row_scales = Hkv * kD / kBlock;
  // Each tile is read through buffer resources that start at the tile and end
  // at the cache's end (no bytes for a tile that does not exist), so a lane's
  // offsets are the same for every tile and the keys past T read zeros.
  auto tile_rsrc = [&](const void* base, int k, int row_bytes) {
    const bool live = exists(k);
    const uint32_t off = live ? (uint32_t)phys(k) * kTileKeys * row_bytes : 0u;
    const uint32_t n = live ? (uint32_t)T * row_bytes - off : 0u;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const unsigned char*>(base) + off), 0, n,
                                             kRsrcWord3);
  };
  uint32_t kvo[2], kso[2], vvo[4], vso[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    kvo[h] = (uint32_t)((16 * h + c) * row_codes + head * (kD / 2) + 32 * grp);
    kso[h] = (uint32_t)(((16 * h + c) * row_scales + head * (kD / kBlock) + 2 * grp) * 2);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vvo[i] = (uint32_t)((8 * i + (lane & 7)) * row_codes + head * (kD / 2) + kBlockBytes * (lane >> 3));
    vso[i] = (uint32_t)(((8 * i + (lane & 7)) * row_scales + head * (kD / kBlock) + (lane >> 3)) * 2);
  }

  // K of half h: 32 code bytes (8 words) and 2 block scales of key 16 h + c.
  // V load i: the 16 code bytes (one block) of key 8 i + (l & 7), block
  // l >> 3, and its scale (8 whole 128-byte lines per load instruction).
  uint4 kc[2][2], vc[4];
  uint32_t ksc[2], vsc[4];
  auto load_k = [&](int k) {
    const __amdgpu_buffer_rsrc_t rkc = tile_rsrc(k_codes, k, row_codes);
    const __amdgpu_buffer_rsrc_t rks = tile_rsrc(k_scales, k, row_scales * 2);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rkc, kvo[h], 16 * i, 0);
        kc[h][i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
      ksc[h] = __builtin_amdgcn_raw_buffer_load_b32(rks, kso[h], 0, 0);
    }
  };
  auto load_v = [&](int k) {
    const __amdgpu_buffer_rsrc_t rvc = tile_rsrc(v_codes, k, row_codes);
    const __amdgpu_buffer_rsrc_t rvs = tile_rsrc(v_scales, k, row_scales * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rvc, vvo[i], 0, 0);
      vc[i] = make_uint4(v[0], v[1], v[2], v[3]);
      vsc[i] = __builtin_amdgcn_raw_buffer_load_b16(rvs, vso[i], 0, 0);
    }
  };
  auto word = [](const uint4 (&v)[2], int i) {
    const uint4 x = v[i >> 2];
    const int j = i & 3;
    return j == 0 ? x.x : j == 1 ? x.y : j == 2 ? x.z : x.w;
  };
  auto bq = [&](int rt, int j) -> h8 {
    if constexpr (RT == 1) return as_h8(bq1[j]);
    else return as_h8(qt[(rt * 8 + j) * 64 + lane]);
  };

  // the last position query row 16 rt + c may see (rows past R: every key)
  int lim[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + c;
    lim[rt] = r < R ? T - M + r / G : T - 1;
  }
  const float c2 = 1.4426950408889634f / 16.0f;   // log2(e) / sqrt(D)

  f4 o[RT][16];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[rt][dt] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegBig;
    l_run[rt] = 0.f;
  }

  // V tile addresses.  Row writes: V load i of lane (u = l & 7, b = l >> 3)
  // fills chunks 4 b + w of row 8 i + u: (wr + 4096 i) ^ 16 w.  Transposing
  // reads: lane (c, grp) addresses row 4 grp + c / 4 (+ 16 for the second
  // read), chunk 2 dt + (c % 4) / 2, half c % 2, which is
  // (rd ^ 32 (dt % 8)) + 256 (dt / 8) (+ 8192).
  const int vt = kQtBytes + wave * kVTile;
  const int wr = vt + (lane & 7) * kVRow + 16 * ((4 * (lane >> 3)) ^ vt_swizzle(lane & 7));
  const int trow = 4 * grp + (c >> 2);
  const int rd = vt + trow * kVRow + 16 * (((c & 3) >> 1) ^ vt_swizzle(trow)) + 8 * (c & 1);
  int wrw[4], rdl[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) wrw[w] = wr ^ (16 * w);
#pragma unroll
  for (int dl = 0; dl < 8; ++dl) rdl[dl] = rd ^ (32 * dl);
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  lds_u8* const lds3 = (lds_u8*)lds;

  auto process = [&](int k) {
    const int t0 = phys(k) * kTileKeys;
    // ---- V: dequantize this lane's 4 blocks into the wave's LDS tile ------
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sb = vsc[i] & 0xFFFFu;
      const h2 d2 = as_h2(sb | (sb << 16));
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t cw = w == 0 ? vc[i].x : w == 1 ? vc[i].y : w == 2 ? vc[i].z : vc[i].w;
        const uint4 p = dequant8(cw, d2);
        *reinterpret_cast<uint4*>(lds + wrw[w] + 4096 * i) = p;
      }
    }
    __builtin_amdgcn_sched_barrier(0);            // the next V codes reuse these registers
    load_v(k + kWaves);

    // ---- scores S^T[16 h + 4 grp + i, 16 rt + c] ----------------------------
    f4 s[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) s[rt][0] = s[rt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t sb = j < 4 ? (ksc[h] & 0xFFFFu) : (ksc[h] >> 16);
        const uint4 a = dequant8(word(kc[h], j), as_h2(sb | (sb << 16)));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          s[rt][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(a), bq(rt, j), s[rt][h], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    load_k(k + kWaves);

    // ---- V^T operands of the first value products (read ahead) -------------
    auto load_a = [&](int dt) {
      const int base = rdl[dt & 7] + 256 * (dt >> 3);
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(lds3 + base));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(lds3 + base + 16 * kVRow));
      return __builtin_bit_cast(h8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    h8 av[4];
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) av[dt] = load_a(dt);
    __builtin_amdgcn_sched_barrier(0);

    // ---- softmax (base 2), lazy running max ---------------------------------
    float sv[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 8; ++v) sv[rt][v] = s[rt][v >> 2][v & 3] * c2;
    if (t0 + kTileKeys - 1 > T - M) {              // the tile reaches past some row's limit
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int t = t0 + 16 * (v >> 2) + 4 * grp + (v & 3);
          if (t > lim[rt]) sv[rt][v] = -__builtin_inff();
        }
    }
    bool grow = false;
    float mx[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      mx[rt] = sv[rt][0];
#pragma unroll
      for (int v = 1; v < 8; ++v) mx[rt] = fmaxf(mx[rt], sv[rt][v]);
      grow = grow || mx[rt] > m_run[rt] + kRescaleGap;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float m_new = fmaxf(m_run[rt], halves_max(rows16_max(mx[rt])));
        const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_new);
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) o[rt][dt] *= alpha;
        l_run[rt] *= alpha;
        m_run[rt] = m_new;
      }
    }
    uint4 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float p[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        p[v] = __builtin_amdgcn_exp2f(sv[rt][v] - m_run[rt]);
        l_run[rt] += p[v];
      }
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2 t2 = {(_Float16)p[2 * i], (_Float16)p[2 * i + 1]};
        pk[i] = as_u32(t2);
      }
      pb[rt] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- O^T[d, r] += V^T[d, t] P^T[t, r] -----------------------------------
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      if (dt + 3 < 16) av[(dt + 3) & 3] = load_a(dt + 3);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[dt & 3], as_h8(pb[rt]), o[rt][dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int k = wave;                                 // this wave's tiles: k, k + 8, ... of the slice
  if (exists(k)) {
    load_k(k);
    load_v(k);
  }
#pragma unroll 1
  for (; exists(k); k += kWaves) process(k);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) l_run[rt] = halves_sum(rows16_sum(l_run[rt]));   // the row's 4 lanes

  // ---- combine the 8 waves in LDS (the V tiles are free now) ----------------
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);             // [wave][rt][dt][lane] float4s
  float* mxs = red + 4 * RT * 16 * 64 * 4;                // [wave][32 rows]
  float* lsum = mxs + kWaves * 32;                        // [wave][32 rows]
  if (grp == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) mxs[wave * 32 + 16 * rt + c] = m_run[rt];
  }
  __syncthreads();
  float m_all[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_all[rt] = kNegBig;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m_all[rt] = fmaxf(m_all[rt], mxs[w * 32 + 16 * rt + c]);
    const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_all[rt]);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[rt][dt] *= alpha;
    l_run[rt] *= alpha;
  }
#pragma unroll
  for (int half = kWaves / 2; half >= 1; half >>= 1) {
    __syncthreads();
    if (wave >= half && wave < 2 * half) {
      float4* dst = reinterpret_cast<float4*>(red) + (size_t)(wave - half) * RT * 16 * 64;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < 16; ++dt)
          dst[(rt * 16 + dt) * 64 + lane] = make_float4(o[rt][dt][0], o[rt][dt][1], o[rt][dt][2], o[rt][dt][3]);
      if (grp == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) lsum[(wave - half) * 32 + 16 * rt + c] = l_run[rt];
      }
    }
    __syncthreads();
    if (wave < half) {
      const float4* src = reinterpret_cast<const float4*>(red) + (size_t)wave * RT * 16 * 64;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
          const float4 f = src[(rt * 16 + dt) * 64 + lane];
          o[rt][dt][0] += f.x;
          o[rt][dt][1] += f.y;
          o[rt][dt][2] += f.z;
          o[rt][dt][3] += f.w;
        }
        l_run[rt] += lsum[wave * 32 + 16 * rt + c];
      }
    }
  }

  // ---- wave 0 writes this slice's partial (rows < R) -------------------------
  // D row 4 grp + i of product dt is position 16 dt + 4 grp + i of the V tile
  // row: channel 16 dt + 8 (grp / 2) + 2 (grp % 2) + (0, 4, 1, 5)[i].
  if (wave == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = 16 * rt + c;
      if (r < R) {
        const size_t row = ((size_t)split * Hkv + head) * R + r;
        float* po = part_o + row * kD + 8 * (grp >> 1) + 2 * (grp & 1);
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
          *reinterpret_cast<float2*>(po + 16 * dt) = make_float2(o[rt][dt][0], o[rt][dt][2]);
          *reinterpret_cast<float2*>(po + 16 * dt + 4) = make_float2(o[rt][dt][1], o[rt][dt][3]);
        }
        if (grp == 0) {
          part_ml[2 * row] = m_all[rt];
          part_ml[2 * row + 1] = l_run[rt];
        }
      }
    }
  }
}

// ---- kernel 2: merge the slices -------------------------------------------
// grid (H_kv * R, D / 64), 256 threads: thread (ss, dd) takes channel
// 64 blockIdx.y + dd of slices ss, ss + 4, ... with its own running max (one
// batch of loads in flight for up to 64 slices per part); the four parts are
// then combined in a fixed order.
constexpr int kMergeParts = 4;
__global__ void __launch_bounds__(256)
attn_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                  uint16_t* __restrict__ out, int M, int Hq, int Hkv, int S) {
  __shared__ float m_s[kMergeParts][64], l_s[kMergeParts][64], a_s[kMergeParts][64];
  const int G = Hq / Hkv;
  const int R = M * G;
  const int g = blockIdx.x / R;
  const int r = blockIdx.x - g * R;
  const int ss = threadIdx.x >> 6, dd = threadIdx.x & 63;
  const int d = 64 * blockIdx.y + dd;
  const size_t stride = (size_t)Hkv * R;          // rows between consecutive slices
  const float* ml = part_ml + 2 * ((size_t)g * R + r);
  const float* po = part_o + ((size_t)g * R + r) * kD + d;
  float m = kNegBig, l = 0.f, acc = 0.f;
  for (int s0 = ss; s0 < S; s0 += kMergeParts * kMergeBatch) {
    float ov[kMergeBatch], mv[kMergeBatch], lv[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int s = min(s0 + kMergeParts * i, S - 1);
      ov[i] = po[(size_t)s * stride * kD];
      mv[i] = ml[2 * s * stride];
      lv[i] = ml[2 * s * stride + 1];
    }
    float bm = m;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (s0 + kMergeParts * i < S) bm = fmaxf(bm, mv[i]);
    const float sc = __builtin_amdgcn_exp2f(m - bm);
    l *= sc;
    acc *= sc;
    m = bm;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i)
      if (s0 + kMergeParts * i < S) {
        const float w = __builtin_amdgcn_exp2f(mv[i] - m);
        l += lv[i] * w;
        acc += ov[i] * w;
      }
  }
  m_s[ss][dd] = m;
  l_s[ss][dd] = l;
  a_s[ss][dd] = acc;
  __syncthreads();
  if (ss == 0) {
    float mt = m_s[0][dd];
#pragma unroll
    for (int i = 1; i < kMergeParts; ++i) mt = fmaxf(mt, m_s[i][dd]);
    float a = 0.f, lt = 0.f;
#pragma unroll
    for (int i = 0; i < kMergeParts; ++i) {
      const float w = __builtin_amdgcn_exp2f(m_s[i][dd] - mt);
      a += a_s[i][dd] * w;
      lt += l_s[i][dd] * w;
    }
    const int mq = r / G, hq = g * G + r % G;
    out[((size_t)mq * Hq + hq) * kD + d] = __half_as_ushort(__float2half_rn(a / lt));
  }
}

}  // namespace

int attn_splits(int M, int Hq, int Hkv, int64_t T) {
  (void)M;
  (void)Hq;
  const int64_t ntiles = (T + kTileKeys - 1) / kTileKeys;
  // about one 8-wave workgroup per CU (256), each wave with at least one tile
  int64_t s = (ntiles + kWaves - 1) / kWaves;
  const int64_t cap = Hkv >= 256 ? 1 : 256 / Hkv;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int)s;
}

size_t attn_ws_bytes(int M, int Hq, int Hkv, int64_t T) {
  const int S = attn_splits(M, Hq, Hkv, T);
  const size_t rows = (size_t)S * Hkv * M * (Hq / Hkv);
  return ((rows * kD * sizeof(float) + 255) & ~(size_t)255) + rows * 2 * sizeof(float);
}

hipError_t launch_attn_decode(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                              const uint8_t* v_codes, const uint16_t* v_scales, uint16_t* out, int M,
                              int Hq, int Hkv, int64_t T, void* ws, hipStream_t s) {
  const int S = attn_splits(M, Hq, Hkv, T);
  const int64_t ntiles = (T + kTileKeys - 1) / kTileKeys;
  const int tps = (int)((ntiles + S - 1) / S);
  const size_t rows = (size_t)S * Hkv * M * (Hq / Hkv);
  float* part_o = reinterpret_cast<float*>(ws);
  float* part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                            ((rows * kD * sizeof(float) + 255) & ~(size_t)255));
  // R = M * G query rows per K/V head: one 16-row tile up to 16, else two.
  const int R = M * (Hq / Hkv);
  if (R <= 16)
    hipLaunchKernelGGL(attn_partial_kernel<1>, dim3(S, Hkv), dim3(kThreads), 0, s, q, k_codes, k_scales, v_codes,
                       v_scales, part_o, part_ml, M, Hq, Hkv, (int)T, tps);
  else
    hipLaunchKernelGGL(attn_partial_kernel<2>, dim3(S, Hkv), dim3(kThreads), 0, s, q, k_codes, k_scales, v_codes,
                       v_scales, part_o, part_ml, M, Hq, Hkv, (int)T, tps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(Hkv * M * (Hq / Hkv), kD / 64), dim3(256), 0, s, part_o, part_ml,
                     out, M, Hq, Hkv, S);
  return hipGetLastError();
}

}  // namespace q4w
