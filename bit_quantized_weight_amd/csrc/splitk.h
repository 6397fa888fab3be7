// Deterministic split-K fixup shared by the skinny kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace q4w {

// Sum of the S fp32 partials p[0], p[stride], ..., p[(S-1) stride] in slice
// order.  The partials were written by other workgroups (possibly on other
// XCDs) with agent-scope stores, so they are read with agent-scope loads;
// loads are issued eight at a time before any of them is added, so the
// fixup costs about one memory latency per eight slices instead of one per
// slice.
__device__ __forceinline__ float sum_partials(const float* p, size_t stride, int S) {
  float s = 0.f;
  for (int sp = 0; sp < S; sp += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = min(sp + i, S - 1);   // in range; extra lanes are masked below
      v[i] = __hip_atomic_load(p + (size_t)idx * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (sp + i < S) s += v[i];
  }
  return s;
}

}  // namespace q4w
