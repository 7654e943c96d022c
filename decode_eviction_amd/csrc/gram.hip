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
// Work-group: 8 waves (two per SIMD), 256 rows resident in registers (each
// row group of 64 rows is held by two waves that split every column block).
// Columns stream through LDS 128 keys at a time in a ring of three blocks,
// with direct global->LDS loads issued two blocks ahead; each wave keeps two
// accumulator sets so the fp32 epilogue of one tile runs between the
// matrix-core instructions of the next.  The last step combines R with the
// importance from k_pool into Z = lambda I - (1-lambda) R.
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

// s_waitcnt immediates (gfx9 encoding): wait until at most N vector memory
// operations of this wave are outstanding; LDS/scalar counters untouched.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

template <typename E, int D>
__global__ __launch_bounds__(512, 1) void k_gram(GramParams p) {
  using G = Geo<E, D>;
  constexpr int NC = G::kNC;
  constexpr int RB = G::kRowBytes;
  constexpr int CPR = G::kChunks;        // 16-byte chunks per key
  constexpr int ROWS = 256;              // rows per work-group (4 row groups x 64)
  constexpr int COLS = 128;              // columns per step (2 column groups x 64)
  constexpr int STAGE = COLS * RB;       // one staged key block, unpadded
  constexpr int NBUF = 3 * STAGE <= 96 * 1024 ? 3 : 2;  // ring: current block + NBUF-1 ahead
  constexpr int AHEAD = NBUF - 1;
  constexpr int PER = COLS * CPR / 512;  // 16-byte key chunks each thread streams per step
  constexpr int VM_STEP = PER + 1;       // vector memory operations per thread per step
  constexpr int RED = 65;                // padded row stride of the final reduction
  constexpr int KBYTES = NBUF * STAGE;
  constexpr int HOFF = ROWS * RED * 4;   // LDS histogram after the reduction buffer
  constexpr int LDSB = KBYTES > HOFF + kHistBins * 4 ? KBYTES : HOFF + kHistBins * 4;
  __shared__ __attribute__((aligned(16))) char lds_raw[LDSB];
  __shared__ __attribute__((aligned(16))) float wcol[NBUF][COLS];
  __shared__ float rowss[ROWS];

  const int nrb = (p.cap + ROWS - 1) / ROWS;
  const int W = xcd_major(blockIdx.x, nrb * p.hkv * p.b);
  const int rb = W % nrb, hh = W / nrb;
  const int h = hh % p.hkv, bi = hh / p.hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const int rg = wave >> 1, cg = wave & 1;
  const int n = min(p.lengths[bi], p.cap);
  const int r0 = rb * ROWS;
  if (r0 >= n) return;
  const long head = (long)bi * p.hkv + h;
  const char* kb = p.k + head * (long)p.cap * RB;
  const float* wv = p.inv_norm + head * (long)p.wstride;

  Frag<NC> af[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = r0 + rg * 64 + 32 * rt + l32;
    load_frag<E, D>(af[rt], kb, row, row < n, hf);
    if (cg == 0) {
      float ss = frag_sumsq<E, NC>(af[rt]);
      ss += xor32(ss);
      if (hf == 0) rowss[rg * 64 + 32 * rt + l32] = ss;
    }
  }

  // LDS layout of a staged block: key r, chunk c at 16-byte slot
  // r*CPR + (c ^ (r % CPR)); the XOR swizzle makes the 32 keys of a fragment
  // read hit distinct banks without padding.  The direct global->LDS loads
  // write lane l of a wave instruction to slot (instruction base + l), so each
  // lane fetches the chunk that belongs in its slot.
  int srow[PER], soff[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int P = it * 512 + tid, r = P / CPR, c = (P % CPR) ^ (r & (CPR - 1));
    srow[it] = r;
    soff[it] = c * 16;
  }
  // Columns past n are clamped to key n-1 (finite data); their weights are 0.
  auto stream = [&](int c0, int buf) {
    const bool full = c0 + COLS <= n;
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int row = full ? c0 + srow[it] : min(c0 + srow[it], n - 1);
      const char* src = kb + (long)row * RB + soff[it];
      char* dst = lds_raw + buf * STAGE + (it * 512 + wave * 64) * 16;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
    // weights: each wave streams one half of the block's 128 (the four copies agree)
    const float* wsrc = wv + c0 + (wave & 1) * 64 + lane;
    float* wdst = &wcol[buf][(wave & 1) * 64];
    __builtin_amdgcn_global_load_lds(wsrc, (__attribute__((address_space(3))) void*)wdst, 4, 0, 0);
  };

  int rdoff[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) rdoff[j] = ((2 * j + hf) ^ (l32 & (CPR - 1))) * 16;
  int colrb[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) colrb[ct] = (cg * 64 + 32 * ct + l32) * RB;

  float rsum[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) rsum[rt][i] = 0.f;

  // Two accumulator sets: the fp32 epilogue of one column tile is issued
  // between the matrix-core instructions of the next tile.
  f32x16_t acc_a[2], acc_b[2];
  float w_b = 0.f;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_b[rt][i] = 0.f;
  auto tile = [&](int buf, int ct, f32x16_t (&acc)[2]) {
    Frag<NC> bfr;
    const char* base = lds_raw + buf * STAGE + colrb[ct];
#pragma unroll
    for (int j = 0; j < NC; ++j) bfr.c[j] = *reinterpret_cast<const u32x4_t*>(base + rdoff[j]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][i] = 0.f;
      acc[rt] = mfma_tile<E, NC>(af[rt], bfr, acc[rt]);
    }
    return wcol[buf][cg * 64 + 32 * ct + l32];
  };
  auto fold = [&](const f32x16_t (&acc)[2], float w) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) rsum[rt][i] = fmaf(acc[rt][i], w, rsum[rt][i]);
  };

  // The ring always issues one block per step so that the wait count is a
  // constant: past the last block it re-streams the last block into the
  // buffer no later step reads.
  const int nsteps = (n + COLS - 1) / COLS;
  constexpr int VM_KEEP = (AHEAD - 1) * VM_STEP;  // loads allowed in flight at a step's end
#pragma unroll
  for (int a = 0; a < AHEAD; ++a) stream(min(a, nsteps - 1) * COLS, a);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_KEEP));
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st % NBUF;
    stream(min(st + AHEAD, nsteps - 1) * COLS, (st + AHEAD) % NBUF);
    const float w_a = tile(buf, 0, acc_a);
    fold(acc_b, w_b);
    w_b = tile(buf, 1, acc_b);
    fold(acc_a, w_a);
    if constexpr (NC == 8 && E::kBytes == 2) {
      // 32 MFMAs, each followed by two of the 64 epilogue FMAs
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    }
    // block st+1 has landed once only the newer blocks may still be in flight
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_KEEP));
    __syncthreads();
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  fold(acc_b, w_b);

  // row sums: lane (hf, l32) of wave (rg, cg) holds rows rg*64 + 32rt + tile_row(i, hf)
  float* red = reinterpret_cast<float*>(lds_raw);
  uint32_t* lh = reinterpret_cast<uint32_t*>(lds_raw + HOFF);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      red[(rg * 64 + 32 * rt + tile_row(i, hf)) * RED + cg * 32 + l32] = rsum[rt][i];
  if (p.hist)
    for (int t = tid; t < kHistBins; t += 512) lh[t] = 0u;
  __syncthreads();
  if (tid < ROWS) {
    const int j = r0 + tid;
    if (j < n) {
      float s = 0.f;
      for (int l = 0; l < 64; ++l) s += red[tid * RED + l];
      const float ss = rowss[tid];
      const float inv = inv_norm_of(ss);
      const float inv_nm1 = n > 1 ? 1.0f / (float)(n - 1) : 0.f;
      const float red_j = (inv * s - inv * inv * ss) * inv_nm1;
      const long o = head * p.cap + j;
      if (p.r_out) p.r_out[o] = red_j;
      const float z = p.lambda * p.i_in[o] - (1.0f - p.lambda) * red_j;
      p.z_out[o] = z;
      if (p.hist) atomicAdd(&lh[hist_bin(score_key(z))], 1u);
    }
  }
  if (p.hist) {
    __syncthreads();
    for (int t = tid; t < kHistBins; t += 512)
      if (lh[t]) atomicAdd(&p.hist[head * kHistBins + t], lh[t]);
  }
}

template <typename E, int D>
static hipError_t gram_t(const GramParams& p, hipStream_t s, Trace* tr) {
  const int blocks = (p.cap + 255) / 256 * p.hkv * p.b;
  return launch_k(k_gram<E, D>, dim3(blocks), dim3(512), s, tr, p);
}

hipError_t launch_gram(int dt, int d, const GramParams& p, hipStream_t s, Trace* tr) {
  if (dt == 0) return d == 64 ? gram_t<BF16, 64>(p, s, tr) : gram_t<BF16, 128>(p, s, tr);
  return d == 64 ? gram_t<F32, 64>(p, s, tr) : gram_t<F32, 128>(p, s, tr);
}

}  // namespace kvsel
