// Split-KV plan computed by one workgroup: prefix sums of the clamped
// sequence lengths and the work-item size. It runs either as its own kernel
// or as one extra workgroup of the query-absorption launch that precedes the
// decode (the plan only depends on the lengths).
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace mlra {

// Run by every thread of one workgroup of blockDim.x (a multiple of 64, at
// most 1024) threads; uses 17 ints of LDS. Writes prefix[0..B] and *hdr.
__device__ inline void plan_block(const PlanArgs& a) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < a.B; base += blockDim.x) {
    const int i = base + tid;
    int v = i < a.B ? a.lens[i] : 0;
    v = v < 0 ? 0 : (v > a.max_len ? a.max_len : v);
    int x = v;  // inclusive scan within the wave
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int before = carry_s;
    for (int w = 0; w < wid; ++w) before += wsum[w];
    if (i < a.B) a.prefix[i] = before + x - v;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int w = 0; w < nw; ++w) t += wsum[w];
      carry_s += t;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int total = carry_s;
    a.prefix[a.B] = total;
    int chunk = a.forced_chunk;
    if (chunk <= 0) {
      chunk = (total + a.target_items - 1) / a.target_items;
      if (chunk < kMinChunk) chunk = kMinChunk;
    }
    PlanHeader h;
    h.chunk = chunk;
    h.n_items = total > 0 ? (total + chunk - 1) / chunk : 0;
    h.total = total;
    h.bounds_fail = 0;
    *a.hdr = h;
  }
}

}  // namespace mlra
