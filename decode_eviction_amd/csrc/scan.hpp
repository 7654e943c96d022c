// Work-group scans shared by the selection kernels (select.hip) and the
// fused short-cache step (fused.hip).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace kvsel {

constexpr int kSelWaves = kSelectThreads / kWave;


__device__ __forceinline__ uint32_t lanemask_lt_count(uint64_t m, int lane) {
  return (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

// exclusive prefix sum over the NW*64 threads of the block; returns (prefix, total)
template <int NW = kSelWaves>
__device__ __forceinline__ uint2 block_scan_u32(uint32_t v, uint32_t* wsum, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = wsum[w];
    before += w < wave ? t : 0u;
    total += t;
  }
  __syncthreads();
  return make_uint2(before + x - v, total);
}

}  // namespace kvsel
