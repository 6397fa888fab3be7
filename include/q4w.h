/*
 * q4w.h -- C ABI of the MI355X (gfx950) 4-bit block-quantized weight matmul.
 *
 * Four operations, each from the pages on 4-bit LLM inference:
 *
 *   q4_pack            weight quantization into the 4-bit block format.
 *                      "Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF"
 *                      (page 3), the paragraph naming the public Q4_0 GGUF.
 *   q4_gemv_skinny     the weight-streaming matmul of decode and of
 *                      speculative verification (M = 1 + drafted tokens).
 *                      Same page, the paragraph on decode streaming the
 *                      quantized weights on every step, and the MTP
 *                      n_max = 3 result (an M = 4 verify).
 *   a8w4_gemm_prefill  the A8 prefill route: int8 activations per token per
 *                      64 channels against the 4-bit weights in an int8
 *                      matrix-core contraction.  "Qwen3.8-27B on RTX 4090:
 *                      5,000 tok/s Prefill Reproduced" (page 5), section
 *                      "Why the A8 artifact matters".
 *   q4_attn_decode     the decode-time read of a K/V cache held in the same
 *                      4-bit format.  Page 3, the architecture and bandwidth
 *                      paragraphs (16 full-attention layers with Q4 K and V).
 *
 * Format (the pages name it but do not define it; this is the reading used):
 *   W is [N, K] fp32, row n = output n, K = reduction width.  Y = X . What^T.
 *   Blocks of 32 consecutive weights along K.  Per block an fp16 scale
 *   d = fp16_RNE(fl32(absmax / 7)) and codes
 *   q = clamp(round_half_away(fl32(w / d)), -8, 7), all 0 when d == 0.
 *   codes  : uint8 [N, K/2] row-major; byte j of row n holds code 2j in its
 *            low nibble and code 2j+1 in its high nibble, two's complement.
 *   scales : fp16 bit patterns, uint16 [N, K/32] row-major.
 *   What[n, k] = q[n, k] * d[n, k / 32].
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers (hipMalloc'd or equivalent),
 *     owned by the caller; the library never allocates or frees memory and
 *     keeps no state besides a per-thread copy of the last HIP error and the
 *     static device scratch of q4_gemv_skinny_noalloc (with its address per
 *     device).
 *   - Half-precision values cross the ABI as uint16_t bit patterns.
 *   - `stream` is the caller's HIP stream (NULL = default stream).  Each call
 *     only enqueues work and returns; results are valid once the stream is
 *     synchronized, and inputs must stay alive until then.
 *   - All argument checks run on the host before any HIP call; a failed check
 *     returns a negative status and enqueues nothing.  No C++ exception
 *     crosses the ABI.
 *   - Preconditions that are NOT checked (they would need a device sync):
 *     weights finite with |w| <= 7 * 65504, activations finite.
 *   - Calls that share a workspace must not overlap in time (they race).
 */
#ifndef Q4W_H
#define Q4W_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-valued entry point. */
#define Q4W_OK                     0
#define Q4W_ERR_INVALID_ARG       -1  /* null pointer, negative size, bad split_k */
#define Q4W_ERR_UNSUPPORTED_SHAPE -2  /* M, K outside what the route supports */
#define Q4W_ERR_MISALIGNED        -3  /* a pointer violates the stated alignment */
#define Q4W_ERR_WORKSPACE         -4  /* workspace missing or smaller than required */
#define Q4W_ERR_HIP               -5  /* a HIP call failed; see q4w_last_hip_error() */

/*
 * q4_pack: quantize fp32 weights into codes + scales (format above).
 *   w      [N, K] fp32, 16-byte aligned.
 *   codes  [N, K/2] uint8, 16-byte aligned.  scales [N, K/32] uint16, 2-byte aligned.
 *   K % 32 == 0 (else UNSUPPORTED_SHAPE).  N == 0 or K == 0: nothing to do, OK.
 * Bit-exact with the rule above: IEEE fp32 division (no fast-math), fp16
 * round-to-nearest-even, round half away from zero, clamp to [-8, 7].
 */
int q4_pack(const float* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales,
            hipStream_t stream);

/*
 * q4_gemv_skinny: Y[M, N] = X[M, K] . What^T for 1 <= M <= 16 (decode, and
 *   verification of up to 15 drafted tokens: the 12-token DFlash2 draft
 *   window of page 5, section "DFlash2 reached 282 tok/s on a code prompt",
 *   verifies M = 13 rows).
 *   x      [M, K] fp16, 16-byte aligned.      y [M, N] fp16 (RNE of an fp32
 *   accumulation), 4-byte aligned.            codes/scales as above.
 *   split_k: 0 = library choice, else 1..64 slices of K reduced in a fixed
 *   order (deterministic: the same inputs give bit-identical outputs).
 *   ws / ws_bytes: device workspace of at least q4_gemv_skinny_ws_bytes(M, N,
 *   K, split_k) bytes (0 bytes when that function returns 0; ws may then be
 *   NULL).  Layout: a fixed 256 KiB region of per-tile arrival counters, then
 *   fp32 partial sums.  The workspace must be zero-filled once before its
 *   first use; every completed call leaves the counter region zeroed again,
 *   so one workspace may serve any sequence of shapes (not concurrently).
 *   M outside [1, 16], K % 32 != 0, K > 2^24 or N > 2^19: UNSUPPORTED_SHAPE.
 *   N == 0: OK, nothing enqueued.  K == 0: y is filled with zeros.
 */
size_t q4_gemv_skinny_ws_bytes(int M, int64_t N, int64_t K, int split_k);
int q4_gemv_skinny(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                   uint16_t* y, int M, int64_t N, int64_t K, int split_k,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * q4_gemv_skinny_noalloc: for callers that cannot allocate device memory
 *   (code under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc) and so cannot provide the workspace of q4_gemv_skinny.  Same
 *   arguments, checks and result as q4_gemv_skinny without ws / ws_bytes: the
 *   same plan and kernels run, so the output is bit-identical to
 *   q4_gemv_skinny's for the same inputs.  The split-K workspace is instead a
 *   static device array of Q4W_NOALLOC_SCRATCH_BYTES bytes inside the
 *   library (a 256 KiB counter region, then 8 MiB of fp32 partials: the
 *   default plan of every M <= 16 fits for the projections (K, N) = (5120,
 *   7168), (5120, 5120), (5120, 17408) and (17408, 5120)), which each device
 *   the library runs on holds until the process ends.  Nothing is allocated
 *   or freed.
 *   A plan that needs more than Q4W_NOALLOC_SCRATCH_BYTES (see
 *   q4_gemv_skinny_ws_bytes) returns Q4W_ERR_WORKSPACE before anything is
 *   enqueued.
 *   The first call on a device (with that device current; not under graph
 *   capture) looks up the array's device address and enqueues on `stream`
 *   one small kernel that zeroes its counter region; every completed call
 *   leaves the counters zeroed again and overwrites every partial before
 *   reading it.  All calls on one device share the array: calls that overlap
 *   in time on one device (two streams, two threads) race and give wrong
 *   results.
 */
#define Q4W_NOALLOC_SCRATCH_BYTES (256u * 1024u + 8u * 1024u * 1024u)
int q4_gemv_skinny_noalloc(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                           uint16_t* y, int M, int64_t N, int64_t K, int split_k,
                           hipStream_t stream);

/*
 * a8_quantize_act: per token m and 64-channel group g,
 *   sa[m, g] = fl32(absmax / 127),
 *   xq[m, k] = clamp(round_half_away(fl32(x / sa)), -127, 127), 0 if sa == 0.
 *   x [M, K] fp16 (16-byte aligned), xq [M, K] int8 row-major (16-byte
 *   aligned), sa [M, K/64] fp32 row-major (4-byte aligned).  K % 64 == 0.
 *   M == 0 or K == 0: OK, nothing enqueued.
 */
int a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* sa,
                    hipStream_t stream);

/*
 * a8w4_gemm_prefill: the whole A8 route for any M >= 1:
 *   quantize x as a8_quantize_act does (into the workspace, in a tiled
 *   layout private to the library), form the exact int32 block sums
 *   I[m, n, b] = sum_{k in block b} xq[m, k] * q[n, k] on int8 matrix cores,
 *   and write y[m, n] = fp16_RNE(sum_b sa[m, b/2] * d[n, b] * I[m, n, b])
 *   with the rescale in fp32.
 *   x [M, K] fp16 16-byte aligned; y [M, N] fp16 4-byte aligned.
 *   K % 64 == 0 and K < 2^24 (else UNSUPPORTED_SHAPE: the GEMM's 32-bit buffer
 *   ranges over a 128-row activation tile reach 2^31 at K = 2^24); any M, N >= 1.
 *   ws: at least a8w4_ws_bytes(M, K) bytes, 256-byte aligned.  It holds the
 *   quantized activations and, once M rounded up to 128 reaches 256 rows, a
 *   64 MiB region (arrival counters, then fp32 partial tiles) that the GEMM
 *   uses when its 128 x 128 tiles make a little more than one round of the
 *   GPU's resident workgroups: the K range of every tile is then shared
 *   evenly by all workgroups and the shared tiles are summed in a fixed
 *   order (results are deterministic).  The quantization step zeroes the
 *   counters and every GEMM leaves them zeroed; calls that share a
 *   workspace must not overlap in time.
 *   M == 0 or N == 0: OK, nothing enqueued.  K == 0: y filled with zeros.
 */
size_t a8w4_ws_bytes(int64_t M, int64_t K);
int a8w4_gemm_prefill(const uint16_t* x, const uint8_t* codes, const uint16_t* scales,
                      uint16_t* y, int64_t M, int64_t N, int64_t K,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The A8 route in two calls, for callers that feed one activation matrix to
 * several weight matrices (e.g. the gate and up projections share their
 * input): a8w4_prepare_act quantizes x once into the workspace (the private
 * tiled layout a8w4_gemm_prefill uses internally), and a8w4_gemm_prepared
 * runs the int8 matrix-core GEMM from it.  Together they compute exactly what
 * a8w4_gemm_prefill computes.  Same shape rules, alignments and workspace
 * size (a8w4_ws_bytes(M, K)); the workspace must not be modified between the
 * two calls.  M == 0 or K == 0: prepare enqueues nothing; gemm_prepared with
 * K == 0 fills y with zeros.
 */
int a8w4_prepare_act(const uint16_t* x, int64_t M, int64_t K, void* ws, size_t ws_bytes,
                     hipStream_t stream);
int a8w4_gemm_prepared(const void* ws, const uint8_t* codes, const uint16_t* scales,
                       uint16_t* y, int64_t M, int64_t N, int64_t K, size_t ws_bytes,
                       hipStream_t stream);

/*
 * a8w4_debug_block_acc: test hook.  Same activation quantization and the
 * same int8 matrix-core kernel as a8w4_gemm_prefill, but the epilogue
 * writes the exact int32 block sums acc[m, n, b] (row-major [M, N, K/32])
 * instead of the rescaled result.  Same shape rules and workspace; no
 * scales are read.  Meant for small shapes (the output is M*N*K/32 ints).
 */
int a8w4_debug_block_acc(const uint16_t* x, const uint8_t* codes, int32_t* acc,
                         int64_t M, int64_t N, int64_t K,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * q4_attn_decode: the attention read of one layer's 4-bit K/V cache during
 *   decode and speculative verification.  "Qwen3.8-27B at 256K on a 24GB RTX
 *   PRO 4000 SFF" (page 3): 16 of the 64 layers keep a conventional K/V
 *   cache, held with 4-bit K and V, whose reads grow with the context (the
 *   architecture and bandwidth paragraphs).  For each of the M query tokens
 *   (the last M cache positions: the target token and its drafted tokens)
 *   and each query head h,
 *     o[m, h, :] = sum_t softmax_t(q[m, h, :] . K[t, g, :] / sqrt(D)) V[t, g, :]
 *   over t = 0 .. T - M + m, with g = h / (H_q / H_kv).
 *   Cache layout (the pages name 4-bit K and V but no layout; this is the
 *   reading used): per layer, K and V are each token-major [T, H_kv * D] in
 *   the weight format above (32-element blocks along the head dimension):
 *     k_codes, v_codes   uint8 [T, H_kv * D / 2], 16-byte aligned;
 *     k_scales, v_scales fp16 [T, H_kv * D / 32], 8-byte aligned;
 *   i.e. q4_pack of the fp32 rows [T, H_kv * D] (a step appends its tokens
 *   by packing their rows in place).
 *   q  [M, H_q, D] fp16, 16-byte aligned.  o [M, H_q, D] fp16 (RNE of an
 *   fp32 result), 2-byte aligned.  The kernel dequantizes K and V to fp16
 *   (one rounding of q * d), accumulates scores and outputs in fp32 and
 *   takes the softmax in fp32.
 *   head_dim must be 256; H_q % H_kv == 0; M * (H_q / H_kv) <= 32; M <= T;
 *   T * H_kv * 128 < 2^31 (else UNSUPPORTED_SHAPE).  M, H_q, H_kv < 1 or
 *   T < 0: INVALID_ARG.
 *   ws: at least q4_attn_decode_ws_bytes(...) bytes, 256-byte aligned (the
 *   partial results of the key slices, merged by a second kernel; results
 *   are deterministic).  Calls sharing a workspace must not overlap.
 */
size_t q4_attn_decode_ws_bytes(int M, int n_q_heads, int n_kv_heads, int head_dim, int64_t T);
int q4_attn_decode(const uint16_t* q, const uint8_t* k_codes, const uint16_t* k_scales,
                   const uint8_t* v_codes, const uint16_t* v_scales, uint16_t* o, int M,
                   int n_q_heads, int n_kv_heads, int head_dim, int64_t T, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/*
 * Batched skinny matmuls: one persistent launch computes a whole list of
 * independent y_g = x_g . What_g^T (same M for all, 1 <= M <= 16), e.g. every
 * projection of every layer of one decode step, which the pages' decode
 * streams once per token ("Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF",
 * page 3, the paragraph on weight streaming during decode).  Work items of
 * all matmuls are streamed back to back by resident workgroups, so the
 * weight stream does not drain and refill between matmuls.
 *
 * Work items are 64-row tiles over the whole of K (no split-K); each
 * workgroup keeps the loads of its next chunk of weights in flight while it
 * computes the current one.  Results are deterministic (a fixed summation
 * order: repeated runs are bit-identical) and agree with q4_gemv_skinny to
 * the stated tolerance, not bit for bit (different K split).  The matmuls
 * are independent: no y_g may overlap any x_h, codes_h, scales_h or other
 * y_h of the batch.  A batch should hold many row tiles (N/64 summed over
 * the batch well above the number of CUs); a single small matmul is better
 * served by q4_gemv_skinny.
 *
 * q4w_gemv_desc: one matmul, layouts and alignments as for q4_gemv_skinny;
 *   N >= 1, K >= 32, K % 32 == 0, N <= 2^19, K <= 2^24.
 * q4_gemv_batched_ws_bytes: workspace bytes for the batch (its work table
 *   and every workgroup's list of work items); 0 if a size or shape is
 *   invalid.
 * q4_gemv_batched_plan: a set-up call, not for graph capture.  Checks every
 *   descriptor, deals the work items (64-row tiles x K) to the persistent
 *   workgroups so that each gets about the same rows x K (longest first, to
 *   the least loaded), writes the table and the lists into ws (256-byte
 *   aligned, >= q4_gemv_batched_ws_bytes bytes) and fills *plan.  It synchronizes with the device (blocking copy); the
 *   descriptor array may be freed when it returns.  The workspace then
 *   belongs to the plan until the caller stops using the plan.
 *   Errors: INVALID_ARG (null, count < 1, N or K <= 0), UNSUPPORTED_SHAPE,
 *   MISALIGNED, WORKSPACE, HIP.
 * q4_gemv_batched_run: enqueues the single persistent launch on `stream`
 *   (capturable in a HIP graph); every y_g is complete when the stream
 *   reaches the next command.  Runs of one plan must not overlap in time.
 *   The inputs named by the descriptors are read at run time, so new x_g
 *   contents are picked up by the next run.
 */
typedef struct q4w_gemv_desc {
  const uint16_t* x;       /* [M, K] fp16 */
  const uint8_t* codes;    /* [N, K/2] */
  const uint16_t* scales;  /* [N, K/32] fp16 */
  uint16_t* y;             /* [M, N] fp16 */
  int64_t N;
  int64_t K;
} q4w_gemv_desc;

typedef struct q4w_batched_plan {
  int M;
  int count;
  int total_items;         /* work items of the batch */
  int grid;                /* persistent workgroups launched */
  int variant;             /* kernel variant chosen at plan time */
  void* ws;                /* the workspace holding the table */
} q4w_batched_plan;

size_t q4_gemv_batched_ws_bytes(int M, const q4w_gemv_desc* descs, int count);
int q4_gemv_batched_plan(int M, const q4w_gemv_desc* descs, int count, void* ws,
                         size_t ws_bytes, q4w_batched_plan* plan);
int q4_gemv_batched_run(const q4w_batched_plan* plan, hipStream_t stream);

/*
 * q4w_stream_read: a measurement helper, not a step of the method.  A plain
 *   streaming read of `bytes` bytes at `buf` by `grid` workgroups of `block`
 *   threads, each thread keeping four 16-byte loads in flight, grid-stride
 *   (the whole chip reads one narrow window of the buffer at a time).  It
 *   gives the read rate this GPU reaches for a given launch shape, the
 *   achievable ceiling that the HBM-bound kernels above are measured against
 *   (next to the published 8 TB/s peak).  out (uint32, grid * block / 64
 *   entries, one per wave): out[w * (block / 64) + v] is the XOR of the 32-bit
 *   words that wave v of workgroup w read, a checksum: the XOR of all entries
 *   is the XOR of every word of the buffer.
 *   buf 16-byte aligned (may be NULL when bytes == 0), bytes % 16 == 0 (else
 *   UNSUPPORTED_SHAPE), out 4-byte aligned, 1 <= grid <= 65536,
 *   64 <= block <= 1024 with block % 64 == 0 (else INVALID_ARG).
 */
int q4w_stream_read(const void* buf, size_t bytes, uint32_t* out, int grid, int block, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* q4w_status_str(int status);

/* hipError_t of the last call on this thread that returned Q4W_ERR_HIP. */
int q4w_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4W_H */
