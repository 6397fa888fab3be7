// C ABI of libq4w (declared in include/q4w.h): host-side argument checks,
// workspace sizing and kernel launches.  Every check runs before the first
// HIP call, so each error status can be produced without a GPU.

#include "q4w.h"
#include "q4w_internal.h"

#include <climits>
#include <mutex>
#include <vector>

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return Q4W_OK;
  g_last_hip_error = static_cast<int>(e);
  return Q4W_ERR_HIP;
}

constexpr int64_t kMaxDim = int64_t(1) << 31;  // kernels index rows and columns with 32-bit ints
// The skinny kernel addresses one workgroup's rows (<= 64 x K/2 bytes) through
// a buffer resource with a 32-bit byte range.
constexpr int64_t kMaxSkinnyK = int64_t(1) << 24;
// The A8 GEMM addresses a 128-row activation tile ([4][K/32][64] x 16 B) and
// its chunk offsets with 32-bit buffer sizes and offsets, which stay below
// 2^31 only for K < 2^24.
constexpr int64_t kMaxA8K = (int64_t(1) << 24) - 64;

constexpr int kMaxBatch = 1 << 20;

// Sizes and shapes of a batch (pointers are not looked at).
int check_batch_shapes(int M, const q4w_gemv_desc* d, int count) {
  if (!d || count < 1 || count > kMaxBatch) return Q4W_ERR_INVALID_ARG;
  if (M < 1 || M > q4w::kMaxSkinnyM) return Q4W_ERR_UNSUPPORTED_SHAPE;
  for (int g = 0; g < count; ++g) {
    if (d[g].N <= 0 || d[g].K <= 0) return Q4W_ERR_INVALID_ARG;
    if (d[g].K % q4w::kBlock != 0 || d[g].N > q4w::kMaxSkinnyN || d[g].K > kMaxSkinnyK)
      return Q4W_ERR_UNSUPPORTED_SHAPE;
  }
  return Q4W_OK;
}

q4w::BatchedLayout batch_layout(int M, const q4w_gemv_desc* d, int count,
                                std::vector<int64_t>& N, std::vector<int64_t>& K) {
  N.resize(count);
  K.resize(count);
  for (int g = 0; g < count; ++g) {
    N[g] = d[g].N;
    K[g] = d[g].K;
  }
  return q4w::batched_layout(M, count, N.data(), K.data());
}

// Checks of the skinny entry points, all before any HIP call.  Returns a
// negative status, 1 when there is nothing to do (N == 0), 2 when y is to be
// zero-filled (K == 0), or 0 with *plan filled for a launch.
int skinny_checks(const uint16_t* x, const uint8_t* codes, const uint16_t* scales, const uint16_t* y,
                  int M, int64_t N, int64_t K, int split_k, q4w::SkinnyPlan* plan) {
  if (N < 0 || K < 0 || split_k < 0 || split_k > 64) return Q4W_ERR_INVALID_ARG;
  if (M < 1 || M > q4w::kMaxSkinnyM || K % q4w::kBlock != 0) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (N > q4w::kMaxSkinnyN || K > kMaxSkinnyK) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (N == 0) return 1;
  if (!y) return Q4W_ERR_INVALID_ARG;
  if (!aligned(y, 4)) return Q4W_ERR_MISALIGNED;
  if (K == 0) return 2;
  if (!x || !codes || !scales) return Q4W_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 2)) return Q4W_ERR_MISALIGNED;
  *plan = q4w::plan_skinny(M, N, K, split_k);
  return Q4W_OK;
}

}  // namespace

// ---- scratch of the allocation-free skinny entry point ----------------------
// The split-K workspace of q4_gemv_skinny_noalloc (arrival counters, then fp32
// partials) is this file-scope device array; every device holds its own copy
// until the process ends.  In host code the name `scratch` stands for a
// host-side shadow, never for device memory: the device address is obtained
// with hipGetSymbolAddress, once per device, and only that address is passed
// to kernels.
static_assert(Q4W_NOALLOC_SCRATCH_BYTES > q4w::kCounterRegionBytes, "room for partials");
static_assert(Q4W_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte lines");
static __device__ __align__(256) unsigned char scratch[Q4W_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of `scratch` on the current device.  The first call on a
// device looks the address up and enqueues, on `stream`, a fill kernel that
// zeroes the counter region (every completed skinny call leaves it zeroed
// again, so this is needed once).
hipError_t scratch_on_current_device(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || !aligned(p, 256)) return hipErrorInvalidSymbol;
    e = q4w::launch_fill_zero_u16(static_cast<uint16_t*>(p),
                                  (int64_t)(q4w::kCounterRegionBytes / sizeof(uint16_t)), stream);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int q4_pack(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales,
            hipStream_t stream) {
  if (N < 0 || K < 0) return Q4W_ERR_INVALID_ARG;
  if (K % q4w::kBlock != 0) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (N == 0 || K == 0) return Q4W_OK;
  if (!w || !codes || !scales) return Q4W_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 2)) return Q4W_ERR_MISALIGNED;
  return hip_status(q4w::launch_pack(w, N, K, codes, scales, stream));
}

size_t q4_gemv_skinny_ws_bytes(int M, int64_t N, int64_t K, int split_k) {
  if (M < 1 || M > q4w::kMaxSkinnyM || N <= 0 || N > q4w::kMaxSkinnyN || K <= 0 || K > kMaxSkinnyK ||
      K % q4w::kBlock != 0 || split_k < 0 || split_k > 64)
    return 0;
  return q4w::plan_skinny(M, N, K, split_k).ws_bytes;
}

int q4_gemv_skinny(const uint16_t* x, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                   int M, int64_t N, int64_t K, int split_k, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  q4w::SkinnyPlan p{};
  const int c = skinny_checks(x, codes, scales, y, M, N, K, split_k, &p);
  if (c < 0) return c;
  if (c == 1) return Q4W_OK;
  if (c == 2) return hip_status(q4w::launch_fill_zero_u16(y, int64_t(M) * N, stream));
  if (p.ws_bytes > 0) {
    if (!ws || ws_bytes < p.ws_bytes) return Q4W_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return Q4W_ERR_MISALIGNED;
  }
  return hip_status(q4w::launch_skinny(x, codes, scales, y, M, N, K, p, ws, stream));
}

int q4_gemv_skinny_noalloc(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                           uint16_t* y, int M, int64_t N, int64_t K, int split_k,
                           hipStream_t stream) {
  q4w::SkinnyPlan p{};
  const int c = skinny_checks(x, codes, scales, y, M, N, K, split_k, &p);
  if (c < 0) return c;
  if (c == 1) return Q4W_OK;
  if (c == 2) return hip_status(q4w::launch_fill_zero_u16(y, int64_t(M) * N, stream));
  if (p.ws_bytes > Q4W_NOALLOC_SCRATCH_BYTES) return Q4W_ERR_WORKSPACE;
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    const hipError_t e = scratch_on_current_device(&ws, stream);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(q4w::launch_skinny(x, codes, scales, y, M, N, K, p, ws, stream));
}

int a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* sa,
                    hipStream_t stream) {
  if (M < 0 || K < 0) return Q4W_ERR_INVALID_ARG;
  if (K % q4w::kActGroup != 0) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (M >= kMaxDim || K >= kMaxDim) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || K == 0) return Q4W_OK;
  if (!x || !xq || !sa) return Q4W_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(sa, 4)) return Q4W_ERR_MISALIGNED;
  return hip_status(q4w::launch_act_quant_rowmajor(x, M, K, xq, sa, stream));
}

size_t a8w4_ws_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % q4w::kActGroup != 0) return 0;
  return q4w::a8_ws_bytes(M, K);
}

// Shared checks of the A8 entry points: negative = status to return, 1 = nothing
// to do, 2 = empty reduction (K == 0), 0 = launch.
static int a8_common(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                     bool need_scales, void* out, size_t out_align, int64_t M, int64_t N,
                     int64_t K, void* ws, size_t ws_bytes) {
  if (M < 0 || N < 0 || K < 0) return Q4W_ERR_INVALID_ARG;
  if (K % q4w::kActGroup != 0) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (M >= kMaxDim || N >= kMaxDim || K > kMaxA8K) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0) return 1;  // nothing to do
  if (!out) return Q4W_ERR_INVALID_ARG;
  if (!aligned(out, out_align)) return Q4W_ERR_MISALIGNED;
  if (K == 0) return 2;            // empty reduction
  if (!x || !codes || (need_scales && !scales)) return Q4W_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 16) || (need_scales && !aligned(scales, 2)))
    return Q4W_ERR_MISALIGNED;
  if (!ws || ws_bytes < q4w::a8_ws_bytes(M, K)) return Q4W_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return Q4W_ERR_MISALIGNED;
  return Q4W_OK;
}

int a8w4_gemm_prefill(const uint16_t* x, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                      int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  const int c = a8_common(x, codes, scales, true, y, 4, M, N, K, ws, ws_bytes);
  if (c < 0) return c;
  if (c == 1) return Q4W_OK;
  if (c == 2) return hip_status(q4w::launch_fill_zero_u16(y, M * N, stream));
  hipError_t e = q4w::launch_act_quant_tiled(x, M, K, ws, stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(q4w::launch_a8w4_gemm(ws, codes, scales, y, nullptr, M, N, K, stream));
}

int a8w4_prepare_act(const uint16_t* x, int64_t M, int64_t K, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (M < 0 || K < 0) return Q4W_ERR_INVALID_ARG;
  if (K % q4w::kActGroup != 0) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (M >= kMaxDim || K > kMaxA8K) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || K == 0) return Q4W_OK;
  if (!x) return Q4W_ERR_INVALID_ARG;
  if (!aligned(x, 16)) return Q4W_ERR_MISALIGNED;
  if (!ws || ws_bytes < q4w::a8_ws_bytes(M, K)) return Q4W_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return Q4W_ERR_MISALIGNED;
  return hip_status(q4w::launch_act_quant_tiled(x, M, K, ws, stream));
}

int a8w4_gemm_prepared(const void* ws, const uint8_t* codes, const uint16_t* scales, uint16_t* y,
                       int64_t M, int64_t N, int64_t K, size_t ws_bytes, hipStream_t stream) {
  // the activations were checked by a8w4_prepare_act; pass a stand-in aligned pointer
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(ws);
  const int c = a8_common(xs ? xs : nullptr, codes, scales, true, y, 4, M, N, K,
                          const_cast<void*>(ws), ws_bytes);
  if (c < 0) return c;
  if (c == 1) return Q4W_OK;
  if (c == 2) return hip_status(q4w::launch_fill_zero_u16(y, M * N, stream));
  return hip_status(q4w::launch_a8w4_gemm(ws, codes, scales, y, nullptr, M, N, K, stream));
}

int a8w4_debug_block_acc(const uint16_t* x, const uint8_t* codes, int32_t* acc, int64_t M,
                         int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int c = a8_common(x, codes, nullptr, false, acc, 4, M, N, K, ws, ws_bytes);
  if (c < 0) return c;
  if (c == 1 || c == 2) return Q4W_OK;  // K == 0 has no blocks to write
  hipError_t e = q4w::launch_act_quant_tiled(x, M, K, ws, stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(q4w::launch_a8w4_gemm(ws, codes, nullptr, nullptr, acc, M, N, K, stream));
}

// Shape checks of the attention read (no pointers): negative status or OK.
static int attn_shape(int M, int n_q_heads, int n_kv_heads, int head_dim, int64_t T) {
  if (M < 1 || n_q_heads < 1 || n_kv_heads < 1 || T < 0) return Q4W_ERR_INVALID_ARG;
  if (head_dim != q4w::kAttnHeadDim || n_q_heads % n_kv_heads != 0) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)M * (n_q_heads / n_kv_heads) > q4w::kAttnMaxRows) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (T < M) return Q4W_ERR_UNSUPPORTED_SHAPE;
  // cache rows are addressed with 32-bit byte offsets
  if (T * (int64_t)n_kv_heads * (head_dim / 2) >= (int64_t(1) << 31)) return Q4W_ERR_UNSUPPORTED_SHAPE;
  return Q4W_OK;
}

size_t q4_attn_decode_ws_bytes(int M, int n_q_heads, int n_kv_heads, int head_dim, int64_t T) {
  if (attn_shape(M, n_q_heads, n_kv_heads, head_dim, T) != Q4W_OK) return 0;
  return q4w::attn_ws_bytes(M, n_q_heads, n_kv_heads, T);
}

int q4_attn_decode(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                   const uint8_t* v_codes, const uint16_t* v_scales, uint16_t* o, int M,
                   int n_q_heads, int n_kv_heads, int head_dim, int64_t T, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  const int st = attn_shape(M, n_q_heads, n_kv_heads, head_dim, T);
  if (st != Q4W_OK) return st;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !o) return Q4W_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_scales, 8) ||
      !aligned(v_scales, 8) || !aligned(o, 2))
    return Q4W_ERR_MISALIGNED;
  if (!ws || ws_bytes < q4w::attn_ws_bytes(M, n_q_heads, n_kv_heads, T)) return Q4W_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return Q4W_ERR_MISALIGNED;
  return hip_status(q4w::launch_attn_decode(q, k_codes, k_scales, v_codes, v_scales, o, M, n_q_heads,
                                            n_kv_heads, T, ws, stream));
}

int q4w_stream_read(const void* buf, size_t bytes, uint32_t* out, int grid, int block, hipStream_t stream) {
  if (!out || (!buf && bytes > 0)) return Q4W_ERR_INVALID_ARG;
  if (grid < 1 || grid > 65536 || block < 64 || block > 1024 || block % 64 != 0) return Q4W_ERR_INVALID_ARG;
  if (bytes % 16 != 0) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (!aligned(buf, 16) || !aligned(out, 4)) return Q4W_ERR_MISALIGNED;
  return hip_status(q4w::launch_stream_read(buf, bytes, out, grid, block, stream));
}

const char* q4w_status_str(int status) {
  switch (status) {
    case Q4W_OK: return "OK";
    case Q4W_ERR_INVALID_ARG: return "INVALID_ARG";
    case Q4W_ERR_UNSUPPORTED_SHAPE: return "UNSUPPORTED_SHAPE";
    case Q4W_ERR_MISALIGNED: return "MISALIGNED";
    case Q4W_ERR_WORKSPACE: return "WORKSPACE";
    case Q4W_ERR_HIP: return "HIP";
    default: return "UNKNOWN";
  }
}

int q4w_last_hip_error(void) { return g_last_hip_error; }

size_t q4_gemv_batched_ws_bytes(int M, const q4w_gemv_desc* descs, int count) {
  if (check_batch_shapes(M, descs, count) != Q4W_OK) return 0;
  std::vector<int64_t> N, K;
  return batch_layout(M, descs, count, N, K).total_bytes;
}

int q4_gemv_batched_plan(int M, const q4w_gemv_desc* descs, int count, void* ws, size_t ws_bytes,
                         q4w_batched_plan* plan) {
  if (!plan) return Q4W_ERR_INVALID_ARG;
  const int st = check_batch_shapes(M, descs, count);
  if (st != Q4W_OK) return st;
  for (int g = 0; g < count; ++g) {
    const q4w_gemv_desc& e = descs[g];
    if (!e.x || !e.codes || !e.scales || !e.y) return Q4W_ERR_INVALID_ARG;
    if (!aligned(e.x, 16) || !aligned(e.codes, 16) || !aligned(e.scales, 2) || !aligned(e.y, 4))
      return Q4W_ERR_MISALIGNED;
  }
  std::vector<int64_t> N, K;
  const q4w::BatchedLayout L = batch_layout(M, descs, count, N, K);
  if (L.total_items > INT_MAX) return Q4W_ERR_UNSUPPORTED_SHAPE;
  if (!ws || ws_bytes < L.total_bytes) return Q4W_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return Q4W_ERR_MISALIGNED;
  std::vector<const uint16_t*> x(count), scales(count);
  std::vector<const uint8_t*> codes(count);
  std::vector<uint16_t*> y(count);
  for (int g = 0; g < count; ++g) {
    x[g] = descs[g].x;
    codes[g] = descs[g].codes;
    scales[g] = descs[g].scales;
    y[g] = descs[g].y;
  }
  const bool quad = q4w::batched_quad(count, K.data(), scales.data());
  const int grid = q4w::batched_grid(M, quad, L.total_items);
  if (grid < 1) return hip_status(hipErrorInvalidDeviceFunction);
  // table and per-workgroup item lists, staged on the host and copied once
  std::vector<char> host(L.total_bytes, 0);
  q4w::batched_fill_table(M, count, x.data(), codes.data(), scales.data(), y.data(), N.data(),
                          K.data(), ws, reinterpret_cast<q4w::BatchedGemv*>(host.data()));
  q4w::batched_schedule(count, N.data(), K.data(), grid,
                        reinterpret_cast<uint32_t*>(host.data() + L.table_bytes));
  const hipError_t e = hipMemcpy(ws, host.data(), L.total_bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_status(e);
  plan->M = M;
  plan->variant = quad ? 1 : 0;
  plan->count = count;
  plan->total_items = (int)L.total_items;
  plan->grid = grid;
  plan->ws = ws;
  return Q4W_OK;
}

int q4_gemv_batched_run(const q4w_batched_plan* plan, hipStream_t stream) {
  if (!plan || !plan->ws || plan->M < 1 || plan->M > q4w::kMaxSkinnyM || plan->count < 1 ||
      plan->total_items < 1 || plan->grid < 1 || plan->variant < 0 || plan->variant > 1)
    return Q4W_ERR_INVALID_ARG;
  return hip_status(q4w::launch_batched(plan->M, plan->variant == 1, plan->ws, plan->count,
                                        plan->total_items, plan->grid, stream));
}

}  // extern "C"
