// Redundancy through the Gram matrix on the matrix cores.
//
// R-KV redundancy (QbitAI R-KV article, section "R-KV三步走", redundancy
// scoring from key cosine similarity): R[j] = (1/(n-1)) sum_{i != j} cos(k_i, k_j).
// With w_i = 1/||k_i|| this is
//     R[j] = w_j * ( sum_i w_i (k_i . k_j)  -  w_j ||k_j||^2 ) / (n-1).
// The raw bf16 keys go into the matrix cores (exact products, fp32
// accumulation); the inverse norms are applied in fp32 afterwards, because
// rounding normalised keys to bf16 first would cost about three decimal
// digits of R.  The n x n Gram matrix only ever lives in accumulator
// registers: after each 256 x 128 tile each lane folds its 16 outputs into 16
// running row sums weighted by its column's w_i.
//
// Work-group: 4 waves, 256 rows resident in registers (each wave 64 rows =
// two 32-row tiles); the columns stream through LDS 128 keys at a time,
// double-buffered, with the next block prefetched into registers while the
// matrix cores work on the current one.  The epilogue combines R with the
// importance from k_pool into Z = lambda I - (1-lambda) R.
#include "common.hpp"
#include "kernels.hpp"

namespace kvsel {

template <typename E, int D>
__global__ __launch_bounds__(256) void k_gram(GramParams p) {
  using G = Geo<E, D>;
  constexpr int NC = G::kNC;
  constexpr int RB = G::kRowBytes;
  constexpr int CPR = G::kChunks;       // 16-byte chunks per key
  constexpr int ROWS = 256;
  constexpr int COLS = 128;
  constexpr int LROW = RB + 16;         // padded LDS row
  constexpr int PER = COLS * CPR / 256; // staged chunks per thread
  __shared__ __attribute__((aligned(16))) char lds[2][COLS * LROW];
  __shared__ float wcol[2][COLS];
  __shared__ float rowss[ROWS];

  const int rb = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const int n = min(p.lengths[bi], p.cap);
  const int r0 = rb * ROWS;
  if (r0 >= n) return;
  const long head = (long)bi * p.hkv + h;
  const char* kb = p.k + head * (long)p.cap * RB;
  const float* wv = p.inv_norm + head * p.cap;

  Frag<NC> af[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = r0 + wave * 64 + 32 * rt + l32;
    load_frag<E, D>(af[rt], kb, row, row < n, hf);
    float ss = frag_sumsq<E, NC>(af[rt]);
    ss += xor32(ss);
    if (hf == 0) rowss[wave * 64 + 32 * rt + l32] = ss;
  }

  float rsum[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) rsum[rt][i] = 0.f;

  u32x4_t stage[PER];
  float wstage = 0.f;
  auto gload = [&](int c0) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int cid = it * 256 + tid, r = cid / CPR, ch = cid % CPR, col = c0 + r;
      stage[it] = col < n ? ld16(kb + (long)col * RB + ch * 16) : zero4();
    }
    if (tid < COLS) wstage = c0 + tid < n ? wv[c0 + tid] : 0.f;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int cid = it * 256 + tid, r = cid / CPR, ch = cid % CPR;
      *reinterpret_cast<u32x4_t*>(&lds[buf][r * LROW + ch * 16]) = stage[it];
    }
    if (tid < COLS) wcol[buf][tid] = wstage;
  };

  const int nsteps = (n + COLS - 1) / COLS;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) gload((st + 1) * COLS);
    f32x16_t acc[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rt][ct][i] = 0.f;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      Frag<NC> bfr;
      const char* rp = &lds[buf][(32 * ct + l32) * LROW + hf * 16];
#pragma unroll
      for (int j = 0; j < NC; ++j) bfr.c[j] = *reinterpret_cast<const u32x4_t*>(rp + 32 * j);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[rt][ct] = mfma_tile<E, NC>(af[rt], bfr, acc[rt][ct]);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const float w = wcol[buf][32 * ct + l32];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 16; ++i) rsum[rt][i] = fmaf(acc[rt][ct][i], w, rsum[rt][i]);
    }
    if (st + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  // row sums: lane (hf, l32) holds rows wave*64 + 32rt + tile_row(i, hf), column share l32
  float* red = reinterpret_cast<float*>(&lds[0][0]);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(wave * 64 + 32 * rt + tile_row(i, hf)) * 33 + l32] = rsum[rt][i];
  __syncthreads();
  const int j = r0 + tid;
  if (j < n) {
    float s = 0.f;
    for (int l = 0; l < 32; ++l) s += red[tid * 33 + l];
    const float ss = rowss[tid];
    const float inv = inv_norm_of(ss);
    const float inv_nm1 = n > 1 ? 1.0f / (float)(n - 1) : 0.f;
    const float red_j = (inv * s - inv * inv * ss) * inv_nm1;
    const long o = head * p.cap + j;
    if (p.r_out) p.r_out[o] = red_j;
    p.z_out[o] = p.lambda * p.i_in[o] - (1.0f - p.lambda) * red_j;
  }
}

template <typename E, int D>
static hipError_t gram_t(const GramParams& p, hipStream_t s, Trace* tr) {
  const dim3 grid((p.cap + 255) / 256, p.hkv, p.b);
  return launch_k(k_gram<E, D>, grid, dim3(256), s, tr, p);
}

hipError_t launch_gram(int dt, int d, const GramParams& p, hipStream_t s, Trace* tr) {
  if (dt == 0) return d == 64 ? gram_t<BF16, 64>(p, s, tr) : gram_t<BF16, 128>(p, s, tr);
  return d == 64 ? gram_t<F32, 64>(p, s, tr) : gram_t<F32, 128>(p, s, tr);
}

}  // namespace kvsel
