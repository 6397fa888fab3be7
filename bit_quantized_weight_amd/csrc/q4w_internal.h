// Internal launch interface between the C ABI (q4w_api.hip) and the kernels.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4w {

// ---- 4-bit block format ---------------------------------------------------
constexpr int kBlock = 32;        // weights per block along K
constexpr int kBlockBytes = 16;   // packed codes per block
constexpr int kActGroup = 64;     // activation channels per int8 scale (A8 route)

hipError_t launch_pack(const float* w, int64_t N, int64_t K, uint8_t* codes,
                       uint16_t* scales, hipStream_t s);

// ---- skinny (M <= 16) weight-streaming matmul -----------------------------
constexpr int kMaxSkinnyM = 16;
// Split-K arrival counters: one uint32 per row tile, in a fixed region at the
// start of the workspace.  The smallest row tile is 8 rows, so 65536 counters
// cover N <= 2^19.
constexpr size_t kCounterRegionBytes = 256 * 1024;
constexpr int kMinRowsPerTile = 8;
constexpr int64_t kMaxSkinnyN = int64_t(1) << 19;
static_assert(int64_t(kCounterRegionBytes / 4) * kMinRowsPerTile >= kMaxSkinnyN,
              "one counter per row tile at the largest N");
constexpr int kRouteDot2 = 0;     // VALU dot2 kernel (q4_gemv.hip)
constexpr int kRouteMfma = 1;     // 16x16x32 matrix-core kernel (q4_gemv_mfma.hip)
constexpr int kRouteMfma4 = 2;    // 4x4x4 matrix-core kernel (q4_gemv_mfma4.hip)
constexpr int kMfmaMinM = 8;      // smallest M routed to the 16x16x32 kernel
constexpr int kMfma4MinM = 4;     // M in [kMfma4MinM, kMfmaMinM) takes the 4x4x4 kernel
constexpr int kMfma4SplitM = 3;   // at this M, rows longer than one 4x4x4 slice go there too
constexpr int kMfma4SliceBlocks = 160;   // longest one-slice row of the 4x4x4 kernel (blocks)
struct SkinnyPlan {
  int route;           // kRouteDot2, kRouteMfma or kRouteMfma4
  int rows_per_wg;     // output rows per workgroup
  int row_tiles;       // ceil(N / rows_per_wg)
  int splits;          // K slices
  int blocks_per_split;
  size_t ws_bytes;     // 0 when splits == 1
  size_t counter_bytes;
};
SkinnyPlan plan_skinny(int M, int64_t N, int64_t K, int split_k);
SkinnyPlan plan_skinny_mfma(int M, int64_t N, int64_t K, int split_k);
SkinnyPlan plan_skinny_mfma4(int M, int64_t N, int64_t K, int split_k);
hipError_t launch_skinny_mfma4(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                               uint16_t* y, int M, int64_t N, int64_t K, const SkinnyPlan& p,
                               void* ws, hipStream_t s);
hipError_t launch_skinny_mfma(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                              uint16_t* y, int M, int64_t N, int64_t K, const SkinnyPlan& p,
                              void* ws, hipStream_t s);
hipError_t launch_skinny(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                         uint16_t* y, int M, int64_t N, int64_t K, const SkinnyPlan& p,
                         void* ws, hipStream_t s);

hipError_t launch_fill_zero_u16(uint16_t* y, int64_t count, hipStream_t s);

// ---- batched skinny matmuls (one persistent launch) ------------------------
// Device-side table entry: one matmul of the batch (the streaming kernel
// uses x, codes, scales, y, N, K and item_begin).
struct BatchedGemv {
  const uint16_t* x;
  const uint4* codes;
  const uint16_t* scales;
  uint16_t* y;
  float* partial;       // S x M x N fp32 split-K partials (S > 1)
  uint32_t* counters;   // one arrival counter per row tile (S > 1)
  int N, K, bps, S;
  int item_begin;       // index of this matmul's first work item
  int pad[3];
};
static_assert(sizeof(BatchedGemv) == 80, "table entry layout");

// Workspace layout of a batch: the table, then each persistent workgroup's
// list of work items (uint32 offsets[kMaxBatchedGrid + 1], then the items),
// both 256-byte aligned.
constexpr int kMaxBatchedGrid = 4096;
struct BatchedLayout {
  size_t table_bytes, sched_bytes, total_bytes;
  int64_t total_items;
};
BatchedLayout batched_layout(int M, int count, const int64_t* N, const int64_t* K);
// Deals the items of a batch to `grid` workgroups, longest first, each to the
// least loaded workgroup so far (cost: rows x K), and lists every workgroup's
// items in ascending order.  sched: offsets[grid + 1] then items, as laid out
// in the workspace (host memory, sched_bytes).
void batched_schedule(int count, const int64_t* N, const int64_t* K, int grid, uint32_t* sched);
// Fills `table` (host memory, count entries) for a workspace at device address ws.
void batched_fill_table(int M, int count, const uint16_t* const* x, const uint8_t* const* codes,
                        const uint16_t* const* scales, uint16_t* const* y, const int64_t* N,
                        const int64_t* K, void* ws, BatchedGemv* table);
// Whether every matmul of a batch takes its 4 step scales in one 8-byte load.
bool batched_quad(int count, const int64_t* K, const uint16_t* const* scales);
// Persistent workgroups to launch for a batch of total_items items.
int batched_grid(int M, bool quad, int64_t total_items);
hipError_t launch_batched(int M, bool quad, const void* ws, int count, int total_items, int grid,
                          hipStream_t s);

// ---- attention read of a 4-bit K/V cache (decode) ---------------------------
constexpr int kAttnHeadDim = 256;   // head dimension the kernel is built for
constexpr int kAttnMaxRows = 32;    // M * (H_q / H_kv): query rows of one K/V head
int attn_splits(int M, int Hq, int Hkv, int64_t T);
size_t attn_ws_bytes(int M, int Hq, int Hkv, int64_t T);
// plain streaming read of a device buffer (measurement helper); out[grid]
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int grid, int block,
                              hipStream_t s);
hipError_t launch_attn_decode(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                              const uint8_t* v_codes, const uint16_t* v_scales, uint16_t* out, int M,
                              int Hq, int Hkv, int64_t T, void* ws, hipStream_t s);

// ---- A8 prefill -----------------------------------------------------------
constexpr int kA8TileM = 32;      // rows per MFMA tile of the private activation layout

int64_t a8_padded_rows(int64_t M);
size_t a8_ws_bytes(int64_t M, int64_t K);
hipError_t launch_act_quant_rowmajor(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                                     float* sa, hipStream_t s);
hipError_t launch_act_quant_tiled(const uint16_t* x, int64_t M, int64_t K, void* ws,
                                  hipStream_t s);
hipError_t launch_a8w4_gemm(const void* ws, const uint8_t* codes, const uint16_t* scales,
                            uint16_t* y, int32_t* acc_debug, int64_t M, int64_t N,
                            int64_t K, hipStream_t s);

}  // namespace q4w
