// Deterministic split-K fixup shared by the skinny kernels.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace q4w {

// Fixup of one row tile by the last workgroup to arrive: thread output j
// (j < J) is the sum of its S fp32 partials, added in slice order, so the result does not depend on
// which workgroup arrives last or on C.
//
// The partials were written by other workgroups (possibly on other XCDs)
// with agent-scope stores, so they are read with agent-scope loads.  Slices
// go in chunks of C; the loads of a chunk, for all of the thread's outputs,
// are issued before any of them is added, so a thread waits about
// ceil(S / C) memory latencies whatever its number of outputs.
//
// Slice s of thread output j is p[s stride + off[j]].  jw: outputs 0..jw-1
// are summed.  Every off[j] must be in range (an unwanted output passes 0
// and ignores out[j]).
template <int J, int C>
__device__ __forceinline__ void sum_partials(const float* p, const uint32_t (&off)[J], int jw,
                                             size_t stride, int S, float (&out)[J]) {
#pragma unroll
  for (int j = 0; j < J; ++j) out[j] = 0.f;
  for (int s0 = 0; s0 < S; s0 += C) {
    // Loads are unconditional (past the last slice they re-read it, and
    // outputs past jw read offset 0) so that nothing branches between them.
    float v[J][C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float* slice = p + (size_t)min(s0 + c, S - 1) * stride;   // uniform
#pragma unroll
      for (int j = 0; j < J; ++j)
        v[j][c] = __hip_atomic_load(slice + off[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (j < jw && s0 + c < S) out[j] += v[j][c];
  }
}

// The whole fixup of one row tile: the tile's outputs (m, n), m < M, n in
// [row0, row0 + kRows) with n < N, are numbered o = m kRows + (n - row0) and
// thread t takes o = t, t + kThreads, ...; slice s of output (m, n) is
// partial[(s M + m) N + n].  Writes y[m N + n] as fp16 (round to nearest even).
// kLoads: partial loads a thread keeps in flight.
template <int kRows, int M, int kThreads, int kLoads>
__device__ __forceinline__ void fixup_tile(const float* partial, uint16_t* y, int N, int S, int row0) {
  constexpr int O = kRows * M;
  constexpr int J = (O + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  uint32_t off[J];
  bool live[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int o = tid + j * kThreads;
    const int m = o / kRows;
    const int n = row0 + (o - m * kRows);
    live[j] = o < O && n < N;
    off[j] = live[j] ? (uint32_t)(m * N + n) : 0u;
  }
  // Outputs walked by this wave: o = 64 w + lane + j kThreads < O for lane 0.
  const int first = (tid >> 6) * 64;
  const int jw = first < O ? min(J, (O - first + kThreads - 1) / kThreads) : 0;
  float out[J];
  sum_partials<J, (kLoads / J > 0 ? kLoads / J : 1)>(partial, off, jw, (size_t)M * N, S, out);
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (live[j]) {
      const int o = tid + j * kThreads;
      const int m = o / kRows;
      y[(size_t)m * N + row0 + (o - m * kRows)] = __half_as_ushort(__float2half_rn(out[j]));
    }
}

}  // namespace q4w
