// Tile helpers shared by the score kernels (scores.hip) and the fused
// short-cache step (fused.hip): zeroed accumulators, the lane reduce-scatter
// used for unit-key sums, and the LDS staging of a head's query rows.
#pragma once

#include "common.hpp"

namespace kvsel {

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// One reduce-scatter step over lanes l and l ^ M of a 32-lane half: the
// lane with bit M set keeps the upper half of v (summed with its partner's),
// the other the lower half.
template <int L, int M>
__device__ __forceinline__ void scatter_step(float* v, int l32) {
  const bool up = (l32 & M) != 0;
#pragma unroll
  for (int i = 0; i < L / 2; ++i) {
    const float send = up ? v[i] : v[L / 2 + i];
    const float keep = up ? v[L / 2 + i] : v[i];
    v[i] = keep + __shfl_xor(send, M, 64);
  }
}
// Repeat until PC values are left: with NC chunks per lane the lane then holds
// chunk (l32 / (32 / NC)) of its half, summed over the lanes that differ from
// it in the upper log2(NC) bits of l32.
template <int L, int M, int PC>
__device__ __forceinline__ void scatter_down(float* v, int l32) {
  if constexpr (L > PC) {
    scatter_step<L, M>(v, l32);
    scatter_down<L / 2, M / 2, PC>(v, l32);
  }
}

// The MT*32 query rows of a head are the same for the four waves of a
// work-group.  Where they fit they are copied once into LDS, straight from
// global memory (no registers), and the matrix-core loops read them a chunk
// at a time.  Chunk c of row r sits at slot r*QC + (c ^ (r mod QC)), so the
// 16 lanes of a group reading one chunk of 16 consecutive rows hit distinct
// banks.  Rows >= m lie past the buffer's range and arrive as zeros.
template <typename E, int D, int MT>
struct QStage {
  static constexpr int QC = Geo<E, D>::kChunks;  // 16-byte chunks per row
  static constexpr int SLOTS = MT * 32 * QC;
  static_assert(SLOTS % 256 == 0, "whole work-group copies");
  static constexpr bool kLds = SLOTS * 16 <= 40 * 1024;
  static constexpr int kWords = kLds ? SLOTS : 1;
  // issue the copies; the caller calls landed() and then synchronises
  static __device__ __forceinline__ void issue(u32x4_t* qs, const char* qb, int m, int tid) {
    const auto qr = buf_rsrc(qb, (uint32_t)m * Geo<E, D>::kRowBytes);
#pragma unroll
    for (int u = 0; u < SLOTS / 256; ++u) {
      const int sl = 256 * u + tid, r = sl / QC, c = (sl % QC) ^ (r % QC);
      buf_lds16(qr, qs + 256 * u + (tid & ~63), (uint32_t)r * Geo<E, D>::kRowBytes + 16 * c);
    }
  }
  // Reads back one word of each of this thread's copies before the barrier:
  // the compiler then waits for exactly those copies (not for loads issued
  // after them), and the barrier makes every wave's copies visible.
  static __device__ __forceinline__ void landed(const u32x4_t* qs, int tid) {
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < SLOTS / 256; ++u) x |= reinterpret_cast<const uint32_t*>(qs + 256 * u + tid)[0];
    asm volatile("" ::"v"(x));
  }
  // chunk j of row 32t + l32 for lane half hf (the chunk load_frag puts in c[j])
  static __device__ __forceinline__ u32x4_t chunk(const u32x4_t* qs, int t, int l32, int hf, int j) {
    const int r = 32 * t + l32;
    return qs[r * QC + ((2 * j + hf) ^ (r % QC))];
  }
};

}  // namespace kvsel
