// The pair-block Gram unit for short caches, shared by k_gram_pairs
// (gram.hip) and the launch that runs it beside the importance pooling
// (k_pool_pairs, scores.hip).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace kvsel {

// Map the linear work-group index to (head, row block) so that consecutive
// indices on one XCD (work-groups are dealt to the 8 XCDs round-robin) take
// row blocks of the same head: the CUs of an XCD then sweep the same keys
// through their shared L2.
__device__ __forceinline__ int xcd_major(int L, int total) {
  constexpr int kXcd = 8;
  if (total % kXcd != 0) return L;
  return (L % kXcd) * (total / kXcd) + L / kXcd;
}

// Small caches (cap <= kGramPairCap, bf16, d = 128): one work-group per pair
// of 128-key blocks I <= J, so that even a short cache spreads over many CUs
// (the sweep kernels give a 2K-token cache only nine work-groups per head).
// Fragments come straight from global memory (L2-resident at this size).
// Each wave takes 32 rows of block I and all 128 columns of block J on
// 16x16x32 tiles.  The tile's w-weighted row sums go to slot J of block I's
// keys; its w-weighted column sums (I < J) to slot I of block J's keys; so
// every key ends with one slot per block of the cache, and k_gram_fin adds
// them in slot order (deterministic) and removes the self term.  The grid is
// one-dimensional, (pair, head) units in XCD-major order: the pairs of one
// head run on one XCD and share its keys through that XCD's L2.
__device__ __forceinline__ void gram_pairs_unit(const GramParams& p, int bx) {
  constexpr int RB = 256;  // bytes per key (128 bf16)
  constexpr int BS = 128;  // keys per block
  const int nbh = (p.cap + BS - 1) / BS, npairs = nbh * (nbh + 1) / 2;
  const int unit = xcd_major(bx, npairs * p.hkv * p.b);
  const int hb = unit / npairs, h = hb % p.hkv, bi = hb / p.hkv, tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // pair index -> (I, J): block I owns the pairs J = I .. nbh-1
  int I = 0, rem = unit - hb * npairs;
  while (rem >= nbh - I) {
    rem -= nbh - I;
    ++I;
  }
  const int J = I + rem;
  const int n = clamp_len(p.lengths[bi], p.cap);
  if (J * BS >= n) return;
  const long head = (long)bi * p.hkv + h;
  const char* kb = p.k + head * (long)p.cap * RB;
  float* part = p.part + head * (long)p.nsmax * p.cap;

  // A: rows I*BS + 32 wave + 16 rt + c16; lane chunk g of each 32-dim k-step
  u32x4_t af[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = I * BS + 32 * wave + 16 * rt + c16;
    const char* src = kb + (long)(row < n ? row : 0) * RB + g * 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) af[rt][ks] = row < n ? ld16(src + 64 * ks) : zero4();
  }
  // The weights 1/||k|| of the fold, taken from the fragments themselves (so
  // that the unit depends on nothing but K): the four lanes g of a row hold
  // its 128 dimensions; lane 4g + i then passes row 4g + i of the tile to the
  // lanes that fold it.  Rows past n are zero and weigh 0.
  float wrow[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = dot2_bf16(af[rt][ks][e], af[rt][ks][e], ss);
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float wr = inv_norm_of(ss);
#pragma unroll
    for (int i = 0; i < 4; ++i) wrow[rt][i] = __shfl(wr, 4 * g + i, 64);
  }
  // block J, copied once into LDS (columns past n read as zeros): chunk q of
  // column c at slot 16 c + (q xor (c mod 16)), so the 16 lanes reading one
  // chunk of 16 consecutive columns hit distinct banks
  __shared__ u32x4_t bs[BS * 16];
  {
    const auto rk = buf_rsrc(kb + (long)J * BS * RB, (uint32_t)min(n - J * BS, BS) * RB);
#pragma unroll
    for (int u = 0; u < BS * 16 / 256; ++u) {
      const int sl = 256 * u + tid, c = sl / 16, q = (sl % 16) ^ (c % 16);
      buf_lds16(rk, bs + 256 * u + (tid & ~63), (uint32_t)c * RB + 16 * q);
    }
    // this thread's copies have landed (the compiler waits for exactly
    // these), then every wave's
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < BS * 16 / 256; ++u) x |= reinterpret_cast<const uint32_t*>(bs + 256 * u + tid)[0];
    asm volatile("" ::"v"(x));
    __syncthreads();
  }
  // C[row][col] over the 8 column tiles of block J; lane holds rows 4g + i
  // of each row tile at column c16 of each column tile
  f32x4_t acc[2][8];
  float wcol[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const int cl = 16 * ct + c16;
    u32x4_t bf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bf[ks] = bs[cl * 16 + ((4 * ks + g) ^ c16)];
    {
      // the column's weight from its fragments (columns past n read as zeros)
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = dot2_bf16(bf[ks][e], bf[ks][e], ss);
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      wcol[ct] = inv_norm_of(ss);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[rt][ks]),
                                                    __builtin_bit_cast(bf16x8_t, bf[ks]), c, 0, 0, 0);
      acc[rt][ct] = c;
    }
  }
  // row sums (weights of the columns), summed over the 16 lanes of a row
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) v = fmaf(acc[rt][ct][i], wcol[ct], v);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, 64);
      const int r = I * BS + 32 * wave + 16 * rt + 4 * g + i;
      if (c16 == 0 && r < n) part[(long)J * p.cap + r] = v;
    }
  if (I == J) return;
  // column sums (weights of the rows): over the lane's 8 rows, the 4 lane
  // groups, then the 4 waves in order
  __shared__ float colred[4][BS];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    float v = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) v = fmaf(acc[rt][ct][i], wrow[rt][i], v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (g == 0) colred[wave][16 * ct + c16] = v;
  }
  __syncthreads();
  if (tid < BS) {
    const int col = J * BS + tid;
    const float v = (colred[0][tid] + colred[1][tid]) + (colred[2][tid] + colred[3][tid]);
    if (col < n) part[(long)I * p.cap + col] = v;
  }
}

}  // namespace kvsel
