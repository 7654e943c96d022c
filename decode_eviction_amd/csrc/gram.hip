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
// registers.
//
// Symmetry: G = K K^T, so each unordered pair of 256-key blocks {I, J} is
// computed once.  Row block I takes the diagonal block and the blocks
// J = I + d (mod nb) for d = 1 .. (nb-1)/2, plus d = nb/2 when nb is even and
// I < nb/2; every pair is covered exactly once and all work-groups of a head
// get the same number of blocks.  An off-diagonal tile adds its w-weighted row
// sums to block I (in registers) and its w-weighted column sums to block J:
// those go to a partial buffer, one slot per distance d, so that no two
// work-groups write the same word.  k_gram_fin then adds, per key, its own
// row sums and the slots that have a contributor, in a fixed order
// (deterministic), and forms R and Z = lambda I - (1-lambda) R.
//
// Work-group: 4 waves (one per SIMD, up to 512 registers each), 256 rows
// resident in registers, 64 per wave.  Columns stream through LDS 128 keys at
// a time in a ring of three blocks, with direct global->LDS loads issued two
// blocks ahead.  Each wave sweeps the four 32-column tiles of a block with
// double-buffered B fragments (the next tile's LDS reads overlap this tile's
// matrix-core instructions) and two accumulator sets (a tile's fp32 epilogue
// runs between the matrix-core instructions of the next tile).
#include "common.hpp"
#include "gram_pairs.hpp"
#include "kernels.hpp"

namespace kvsel {

// Blocks of columns (of 256 keys) that row block I computes; see above.
__device__ __forceinline__ int gram_blocks(int I, int nb) {
  return 1 + (nb - 1) / 2 + ((nb % 2 == 0 && I < nb / 2) ? 1 : 0);
}

template <typename E, int D>
__global__ __launch_bounds__(256, 1) void k_gram(GramParams p) {
  using G = Geo<E, D>;
  constexpr int NC = G::kNC;
  constexpr int RB = G::kRowBytes;
  constexpr int NT = 256;                // threads: one wave per SIMD
  constexpr int ROWS = 256;              // rows per work-group: 4 waves x 64
  constexpr int COLS = 128;              // columns per step: 4 tiles of 32
  constexpr int STAGE = COLS * RB;       // one staged key block
  // bf16, d = 128: the explicitly pipelined step below (four ring slots,
  // copies two blocks ahead); other shapes: a plain step loop.
  constexpr bool kFast = NC == 8 && E::kBytes == 2;
  constexpr int NBUF = kFast ? 4 : (3 * STAGE <= 96 * 1024 ? 3 : 2);
  constexpr int AHEAD = kFast ? 2 : NBUF - 1;  // blocks streamed ahead of the one being read
  constexpr int PER = NC;                // 16-byte chunk pairs: global->LDS loads per thread per step
  constexpr int VM_STEP = PER + 1;       // vector memory operations per thread per step
  constexpr int RED = 33;                // padded row stride of the final reduction
  constexpr int KBYTES = NBUF * STAGE;
  constexpr int LDSB = KBYTES > ROWS * RED * 4 ? KBYTES : ROWS * RED * 4;
  __shared__ __attribute__((aligned(16))) char lds_raw[LDSB];
  __shared__ __attribute__((aligned(16))) float wcol[NBUF][COLS];
  __shared__ float colred[3][4][2][COLS];  // column sums per wave (and lane half), by step mod 3

  const int nrb = (p.cap + ROWS - 1) / ROWS;
  const int W = xcd_major(blockIdx.x, nrb * p.hkv * p.b);
  const int rb = W % nrb, hh = W / nrb;
  const int h = hh % p.hkv, bi = hh / p.hkv;
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int r0 = rb * ROWS;
  if (r0 >= n) return;
  const int nb = (n + ROWS - 1) / ROWS;
  const int nsteps = 2 * gram_blocks(rb, nb);
  const long head = (long)bi * p.hkv + h;
  const char* kb = p.k + head * (long)p.cap * RB;
  const float* wv = p.inv_norm + head * (long)p.wstride;
  // first column of step t: block J = rb + t/2 (mod nb), half t%2
  auto col0 = [&](int t) {
    int J = rb + (t >> 1);
    J -= J >= nb ? nb : 0;
    return J * ROWS + (t & 1) * COLS;
  };

  // this wave's 64 rows, resident for the whole sweep (matrix-core operands only)
  Frag<NC> af[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = r0 + wave * 64 + 32 * rt + l32;
    load_frag<E, D>(af[rt], kb, row, row < n, hf);
  }
  // weights of the 32 rows this lane's accumulators cover (0 past n)
  float wrow[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t w4 =
          *reinterpret_cast<const f32x4_t*>(wv + r0 + wave * 64 + 32 * rt + 8 * q + 4 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) wrow[rt][4 * q + e] = w4[e];
    }

  // LDS layout of a staged block: key r, 16-byte chunk c at slot
  // (c / 2) * 256 + 2 r + ((c % 2) ^ sw(r)),  sw(r) = bit 2 of r xor bit 3.
  // A fragment read (32 keys, chunks 2j and 2j+1 for the two lane halves)
  // covers 64 consecutive slots, and sw makes any 8 or 16 consecutive lanes
  // of it hit distinct banks.  The chunk index only moves an immediate
  // offset.  The direct global->LDS loads write lane l of a wave instruction
  // to slot (instruction base + l), so for instruction it thread tid streams
  // key tid / 2, chunk 2 it + ((tid % 2) ^ sw(tid / 2)).
  auto sw = [](int r) { return ((r >> 2) ^ (r >> 3)) & 1; };
  const int schunk_off = ((tid & 1) ^ sw(tid >> 1)) * 16;
  // Columns past n are clamped to key n-1 (finite data); their weights are 0.
  auto stream = [&](int c0, int buf) {
    const int row = min(c0 + (tid >> 1), n - 1);
    const char* src = kb + (long)row * RB + schunk_off;
#pragma unroll
    for (int it = 0; it < PER; ++it) dma_lds16(src + it * 32, lds_raw + buf * STAGE + it * 4096 + wave * 1024);
    // weights: waves 0 and 1 stream the block's 128 (the other two fetch a copy)
    dma_lds4(wv + c0 + (wave & 1) * 64 + lane, &wcol[buf][(wave & 1) * 64]);
  };
  const int rdbase = (2 * l32 + (hf ^ sw(l32))) * 16;  // + 1024 ct + 4096 j

  float rsum[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) rsum[rt][i] = 0.f;

  auto read_b = [&](Frag<NC>& f, int buf, int ct) {
    const char* base = lds_raw + buf * STAGE + rdbase + ct * 1024;
#pragma unroll
    for (int j = 0; j < NC; ++j) f.c[j] = *reinterpret_cast<const u32x4_t*>(base + j * 4096);
  };
  // row sums weighted by the column's w; column sums weighted by the rows' w
  auto fold = [&](const f32x16_t (&acc)[2], float w, int ct, int t) {
    float cs = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        rsum[rt][i] = fmaf(acc[rt][i], w, rsum[rt][i]);
        cs = fmaf(acc[rt][i], wrow[rt][i], cs);
      }
    // each lane half stores the sum over its 16 rows; the flush adds the two
    // halves (no cross-lane exchange here).  t = -1 (the empty carried tile
    // before the first step) writes zeros into the buffer of step 2, which
    // overwrites them before it is flushed.
    colred[(t + 3) % 3][wave][hf][ct * 32 + l32] = cs;
  };
  // column sums of step t to its partial slot (distance t/2; none for the
  // diagonal block); run after the barrier that completes step t
  auto flush = [&](int t) {
    if (tid < COLS && (t >> 1) >= 1) {
      const int c = col0(t) + tid;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += colred[t % 3][w][0][tid] + colred[t % 3][w][1][tid];
      if (c < n) p.part[(head * p.nsmax + (t >> 1) - 1) * (long)p.cap + c] = v;
    }
  };

  // Two accumulator sets: tile ct's fold runs between the matrix-core
  // instructions of tile ct+1; the last tile of a step is folded during the
  // first tile of the next.
  f32x16_t acc[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[1][rt][i] = 0.f;
  float w_carry = 0.f;

  // The ring always issues one block per step so that the wait count is a
  // constant: past the last block it re-streams the last block into the
  // buffer no later step reads.
  constexpr int VM_KEEP = (AHEAD - 1) * VM_STEP;  // loads allowed in flight at a step's end
#pragma unroll
  for (int a = 0; a < AHEAD; ++a) stream(col0(min(a, nsteps - 1)), a);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_KEEP));
  __syncthreads();
  if constexpr (kFast) {
    // Step st reads ring slot st % 4 and copies block st+2 into slot
    // (st+2) % 4, last read in step st-2.  One barrier per step, before
    // tile 3: by then block st+1 has landed (each thread waits for its own
    // copies, the barrier for everyone's), so tile 3 can prefetch tile 0 of
    // block st+1; and every wave is past step st-1, which makes the next
    // step's copy into slot (st+3) % 4 safe.
    // Group j of tile ct: the two matrix-core instructions of tile ct for
    // k-chunk j, one eighth of the previous tile's fold (4 row and 4 column
    // FMAs), the LDS read of chunk j of the next tile into the buffer the
    // previous tile released, and (tile 0) one of the step's copies.  Each
    // group is pinned by a scheduling barrier.
    Frag<NC> bq[2];
    read_b(bq[0], 0, 0);
    for (int st = 0; st < nsteps; ++st) {
      const int buf = st % NBUF, nbuf = (st + 1) % NBUF, dbuf = (st + AHEAD) % NBUF;
      if (st >= 2) flush(st - 2);
      const int c0n = col0(min(st + AHEAD, nsteps - 1));
      const char* src = kb + (long)min(c0n + (tid >> 1), n - 1) * RB + schunk_off;
      const char* dst = lds_raw + dbuf * STAGE + wave * 1024;
      float wt[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) wt[ct] = wcol[buf][ct * 32 + l32];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (ct == 3) {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_KEEP));
          __syncthreads();
        }
        const int cur = ct & 1, prv = cur ^ 1;
        const float wp = ct == 0 ? w_carry : wt[ct - 1];
        float cs0 = 0.f, cs1 = 0.f, cs2 = 0.f, cs3 = 0.f;
        const char* nx = ct < 3 ? lds_raw + buf * STAGE + rdbase + (ct + 1) * 1024
                                : lds_raw + nbuf * STAGE + rdbase;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (ct == 0) {
            dma_lds16(src + j * 32, dst + j * 4096);
            if (j == 0) dma_lds4(wv + c0n + (wave & 1) * 64 + lane, &wcol[dbuf][(wave & 1) * 64]);
          }
          const bf16x8_t bj = __builtin_bit_cast(bf16x8_t, bq[cur].c[j]);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            f32x16_t c = acc[cur][rt];
            if (j == 0) {
#pragma unroll
              for (int i = 0; i < 16; ++i) c[i] = 0.f;
            }
            acc[cur][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, af[rt].c[j]), bj, c, 0, 0, 0);
          }
          const int i0 = 2 * j, i1 = 2 * j + 1;
          rsum[0][i0] = fmaf(acc[prv][0][i0], wp, rsum[0][i0]);
          rsum[0][i1] = fmaf(acc[prv][0][i1], wp, rsum[0][i1]);
          rsum[1][i0] = fmaf(acc[prv][1][i0], wp, rsum[1][i0]);
          rsum[1][i1] = fmaf(acc[prv][1][i1], wp, rsum[1][i1]);
          cs0 = fmaf(acc[prv][0][i0], wrow[0][i0], cs0);
          cs1 = fmaf(acc[prv][0][i1], wrow[0][i1], cs1);
          cs2 = fmaf(acc[prv][1][i0], wrow[1][i0], cs2);
          cs3 = fmaf(acc[prv][1][i1], wrow[1][i1], cs3);
          bq[prv].c[j] = *reinterpret_cast<const u32x4_t*>(nx + j * 4096);
          __builtin_amdgcn_sched_barrier(0);
        }
        const float cs = (cs0 + cs1) + (cs2 + cs3);
        // the previous tile: tile 3 of step st-1 when ct = 0, else tile ct-1
        colred[((ct == 0 ? st - 1 : st) + 3) % 3][wave][hf][(ct == 0 ? 3 : ct - 1) * 32 + l32] = cs;
        if (ct == 3) w_carry = wt[3];
      }
    }
  } else {
    for (int st = 0; st < nsteps; ++st) {
      const int buf = st % NBUF;
      if (st >= 2) flush(st - 2);
      stream(col0(min(st + AHEAD, nsteps - 1)), (st + AHEAD) % NBUF);
      Frag<NC> bq[2];
      read_b(bq[0], buf, 0);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (ct < 3) read_b(bq[(ct + 1) & 1], buf, ct + 1);
        const float w = wcol[buf][ct * 32 + l32];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          f32x16_t z;
#pragma unroll
          for (int i = 0; i < 16; ++i) z[i] = 0.f;
          acc[ct & 1][rt] = mfma_tile<E, NC>(af[rt], bq[ct & 1], z);
        }
        if (ct == 0) fold(acc[1], w_carry, 3, st - 1);
        else fold(acc[(ct - 1) & 1], wcol[buf][(ct - 1) * 32 + l32], ct - 1, st);
        if (ct == 3) w_carry = w;
      }
      // block st+1 has landed once only the newer blocks may still be in flight
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_KEEP));
      __syncthreads();
    }
  }
  // every copy has landed (the ring's last copies overlap the reduction
  // buffer below) before anyone writes it
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  fold(acc[1], w_carry, 3, nsteps - 1);

  // row sums: lane (hf, l32) of wave w holds rows w*64 + 32rt + tile_row(i, hf)
  float* red = reinterpret_cast<float*>(lds_raw);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(wave * 64 + 32 * rt + tile_row(i, hf)) * RED + l32] = rsum[rt][i];
  __syncthreads();
  if (nsteps >= 2) flush(nsteps - 2);
  flush(nsteps - 1);
  {
    const int j = r0 + tid;
    if (j < n) {
      float s = 0.f;
#pragma unroll 8
      for (int l = 0; l < 32; ++l) s += red[tid * RED + l];
      // own row sums minus the self term w_j ||k_j||^2 = 1 / w_j (0 for a zero key)
      const float w = wv[j];
      p.rs[head * p.cap + j] = s - (w > 0.f ? 1.0f / w : 0.f);
    }
  }
}

// The same sweep for bf16 keys of 128 dimensions at large n, over blocks of
// 512 keys, on 16x16x32 matrix-core tiles.  Each wave keeps 128 rows
// resident (eight 16-row tiles) in two sets of 64; a set times a 32-column
// tile is eight independent accumulator chains, so the matrix cores stay
// busy while the other set's fp32 fold runs beside them.  In the 16x16
// output layout a lane holds 4 rows of each tile, so the fold's per-lane row
// sums and row weights take 32 registers each.  Every B fragment read from
// LDS feeds 32 matrix-core instructions, and the per-step copies and barrier
// are spread over a 512-key block.  Weights at positions >= n are replaced by
// 0 in registers (the inverse-norm buffer is only written up to the end of
// the 256-key chunk holding n-1).
//
// 16x16x32 tiles: lane l supplies row (or column) l % 16 and 16-byte chunk
// l / 16 of each 32-dimension k-step; result register i of lane l is row
// 4 (l / 16) + i, column l % 16.  A and B fragments use the same chunk
// assignment, so their dot products cover every dimension exactly once.
__global__ __launch_bounds__(256, 1) void k_gram512(GramParams p) {
  constexpr int RB = 256;                // bytes per key (128 bf16)
  constexpr int ROWS = 512;              // rows per work-group: 4 waves x 128
  constexpr int COLS = 128;              // columns per step: 4 tiles of 32
  constexpr int SPB = ROWS / COLS;       // steps per column block
  constexpr int STAGE = COLS * RB;
  constexpr int NBUF = 4, AHEAD = 2;
  constexpr int NCP = 8;                 // 32-byte chunk pairs per key
  constexpr int VM_STEP = NCP + 1;       // copies per thread per step
  constexpr int VM_KEEP = (AHEAD - 1) * VM_STEP;
  constexpr int RED = 17;                // row-sum partials per row: 16 column residues
  constexpr int CPS = 20;                // column partials: 16 per column (4 waves x 4 lane groups), padded
  constexpr int LDSB = NBUF * STAGE > ROWS * RED * 4 ? NBUF * STAGE : ROWS * RED * 4;
  __shared__ __attribute__((aligned(16))) char lds_raw[LDSB];
  __shared__ __attribute__((aligned(16))) float wcol[NBUF][COLS];
  // [step % 3][column][wave * 4 + lane group]: the 64 lanes of a write hit
  // 64 distinct banks, and a column's 16 partials are four aligned 16-byte reads
  __shared__ __attribute__((aligned(16))) float colred[3][COLS][CPS];

  const int nrb = (p.cap + ROWS - 1) / ROWS;
  const int W = xcd_major(blockIdx.x, nrb * p.hkv * p.b);
  const int rb = W % nrb, hh = W / nrb;
  const int h = hh % p.hkv, bi = hh / p.hkv;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int r0 = rb * ROWS;
  if (r0 >= n) return;
  const int nb = (n + ROWS - 1) / ROWS;
  const int nsteps = SPB * gram_blocks(rb, nb);
  const long head = (long)bi * p.hkv + h;
  const char* kb = p.k + head * (long)p.cap * RB;
  const float* wv = p.inv_norm + head * (long)p.wstride;
  auto col0 = [&](int t) {
    int J = rb + t / SPB;
    J -= J >= nb ? nb : 0;
    return J * ROWS + (t % SPB) * COLS;
  };

  // A fragments: row tile rt (16 rows), k-step j: row l % 16, chunk 4j + l / 16
  u32x4_t af[8][4];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    const int row = r0 + wave * 128 + 16 * rt + c16;
    const char* src = kb + (long)(row < n ? row : 0) * RB + g * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) af[rt][j] = row < n ? ld16(src + 64 * j) : zero4();
  }
  float wrow[8][4];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    const int rbase = r0 + wave * 128 + 16 * rt + 4 * g;
    const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(wv + rbase);
#pragma unroll
    for (int e = 0; e < 4; ++e) wrow[rt][e] = rbase + e < n ? w4[e] : 0.f;
  }
  // A fragments only feed the matrix cores: keep them in accumulation registers
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(af[rt][j]));

  // staged layout and copies as in k_gram: chunk c of key r at 16-byte slot
  // (c/2)*256 + 2r + ((c%2)^sw(r)); a 16-lane group reads one chunk of 16
  // consecutive keys, which covers all 64 banks once
  auto sw = [](int r) { return ((r >> 2) ^ (r >> 3)) & 1; };
  const int schunk_off = ((tid & 1) ^ sw(tid >> 1)) * 16;
  const int rdbase = (g >> 1) * 4096 + (2 * c16 + ((g & 1) ^ sw(c16))) * 16;
  auto stream_all = [&](int c0, int buf) {
    const char* src = kb + (long)min(c0 + (tid >> 1), n - 1) * RB + schunk_off;
#pragma unroll
    for (int it = 0; it < NCP; ++it) dma_lds16(src + it * 32, lds_raw + buf * STAGE + it * 4096 + wave * 1024);
    dma_lds4(wv + c0 + (wave & 1) * 64 + lane, &wcol[buf][(wave & 1) * 64]);
  };
  // B fragment of column half h2 (16 keys) of 32-column tile ct, k-step j
  auto b_addr = [&](int buf, int ct, int h2, int j) {
    return lds_raw + buf * STAGE + rdbase + j * 8192 + ct * 1024 + h2 * 512;
  };
  // column sums of step t: the first 128 threads add a column's 16 partials;
  // the reads are issued early and summed later so their latency overlaps
  // matrix-core work
  f32x4_t fq[4];
  auto flush_issue = [&](int t) {
    if (tid < COLS && t / SPB >= 1) {
#pragma unroll
      for (int k = 0; k < 4; ++k) fq[k] = *reinterpret_cast<const f32x4_t*>(&colred[t % 3][tid][4 * k]);
    }
  };
  auto flush_finish = [&](int t) {
    if (tid < COLS && t / SPB >= 1) {
      const int c = col0(t) + tid;
      const f32x4_t q2 = (fq[0] + fq[1]) + (fq[2] + fq[3]);
      const float v = (q2[0] + q2[1]) + (q2[2] + q2[3]);
      if (c < n) p.part[(head * p.nsmax + t / SPB - 1) * (long)p.cap + c] = v;
    }
  };
  auto flush = [&](int t) {
    flush_issue(t);
    flush_finish(t);
  };

  float rsum[8][4];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rsum[rt][i] = 0.f;
  f32x4_t acc[2][4][2];  // [row set][row tile in the set][column half]
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[s2][rt][h2][i] = 0.f;
  float w_carry[2] = {0.f, 0.f}, csA_carry[2] = {0.f, 0.f};

  // element e = 4 h2 + i of row tile t4 of set S: one row-sum FMA, one
  // column-sum FMA
  auto fold_one = [&](int S, int t4, int e, const float* w, float* cs) {
    const int rt = 4 * S + t4, h2 = e >> 2, i = e & 3;
    rsum[rt][i] = fmaf(acc[S][t4][h2][i], w[h2], rsum[rt][i]);
    cs[2 * h2 + (i & 1)] = fmaf(acc[S][t4][h2][i], wrow[rt][i], cs[2 * h2 + (i & 1)]);
    // pinned beside their product: left free, the compiler sinks a tile's
    // folds past the column flush into one run that the matrix core waits out
    asm volatile("" : "+v"(rsum[rt][i]), "+v"(cs[2 * h2 + (i & 1)]));
  };
  auto fold_part = [&](int S, int t4, const float* w, float* cs) {
#pragma unroll
    for (int e = 0; e < 8; ++e) fold_one(S, t4, e, w, cs);
  };
  // One 16x16x32 product into the accumulator of row tile t4 of set S,
  // column half h2: fragments in accumulation registers, the accumulator in
  // arch registers, where the folds read it.  A product runs 16 cycles, and
  // the SIMD keeps the matrix core fed only while at most two vector
  // instructions sit between consecutive products; the fold is exactly two
  // per product.  The instruction is written out because with the builtin
  // the compiler regroups products and folds (and pads them with wait
  // states), leaving gaps the matrix core waits out.  Written out, the
  // product is invisible to the compiler's hazard tracking, so the schedule
  // itself provides the wait states a vector read of a result needs: every
  // fold reads an accumulator at least seven products and fourteen folds
  // (over 20 instructions) after the product that completed it, and nothing
  // in the loop copies a fragment or an accumulator.
  auto mfma1 = [&](int S, int t4, int h2, int j, const u32x4_t& b) {
    if (j == 0)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
                   : "=v"(acc[S][t4][h2])
                   : "a"(af[4 * S + t4][j]), "a"(b));
    else
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                   : "+v"(acc[S][t4][h2])
                   : "a"(af[4 * S + t4][j]), "a"(b));
  };

#pragma unroll
  for (int a = 0; a < AHEAD; ++a) stream_all(col0(min(a, nsteps - 1)), a);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_KEEP));
  __syncthreads();
  u32x4_t bq[2][4][2];  // [buffer][k-step][column half]
  // column weights of the next step, read once its copies have landed
  float wnext[4][2];
  auto read_w = [&](int b) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) wnext[ct][h2] = wcol[b][ct * 32 + h2 * 16 + c16];
  };
  read_w(0);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) bq[0][j][h2] = *reinterpret_cast<const u32x4_t*>(b_addr(0, 0, h2, j));
  // Ring and barrier as in k_gram: step st reads slot st % 4, copies block
  // st+2 into slot (st+2) % 4 during tile 0, and waits for block st+1 (own
  // copies, then a barrier) before tile 3, which prefetches its first tile.
  // Tile ct: phase A = row set 0 of tile ct with the fold of row set 1 of
  // the previous tile (and that tile's column sums completed); phase B =
  // row set 1 of tile ct with the fold of row set 0 of tile ct.
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st % NBUF, nbuf = (st + 1) % NBUF, dbuf = (st + AHEAD) % NBUF;
    if (st >= 2) flush_issue(st - 2);
    const int c0 = col0(st);
    const int c0n = col0(min(st + AHEAD, nsteps - 1));
    const char* src = kb + (long)min(c0n + (tid >> 1), n - 1) * RB + schunk_off;
    const char* dst = lds_raw + dbuf * STAGE + wave * 1024;
    float wt[4][2];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int c = ct * 32 + h2 * 16 + c16;
        wt[ct][h2] = c0 + c < n ? wnext[ct][h2] : 0.f;
      }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (ct == 3) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM_KEEP));
        __syncthreads();
        read_w(nbuf);
      }
      const int cur = ct & 1, prv = cur ^ 1;
      const int nb_buf = ct < 3 ? buf : nbuf, nct = ct < 3 ? ct + 1 : 0;
      const float* wprev = ct == 0 ? w_carry : wt[ct - 1];
      // phase A
      float b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (ct == 0) {
          dma_lds16(src + (2 * j) * 32, dst + (2 * j) * 4096);
          dma_lds16(src + (2 * j + 1) * 32, dst + (2 * j + 1) * 4096);
          if (j == 0) dma_lds4(wv + c0n + (wave & 1) * 64 + lane, &wcol[dbuf][(wave & 1) * 64]);
        }
        // issue order: one matrix-core instruction, then its two folds,
        // eight times; the next tile's LDS reads after the first
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          mfma1(0, q >> 1, q & 1, j, bq[cur][j][q & 1]);
          fold_one(1, j, q, wprev, b4);
          if (q == 0) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
              bq[prv][j][h2] = *reinterpret_cast<const u32x4_t*>(b_addr(nb_buf, nct, h2, j));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (ct == 0 && st >= 2) flush_finish(st - 2);
      {
        const int slot = ((ct == 0 ? st - 1 : st) + 3) % 3;
        const int pct = ct == 0 ? 3 : ct - 1;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          colred[slot][pct * 32 + h2 * 16 + c16][wave * 4 + g] = csA_carry[h2] + (b4[2 * h2] + b4[2 * h2 + 1]);
      }
      // phase B
      float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          mfma1(1, q >> 1, q & 1, j, bq[cur][j][q & 1]);
          fold_one(0, j, q, wt[ct], a4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      csA_carry[0] = a4[0] + a4[1];
      csA_carry[1] = a4[2] + a4[3];
      if (ct == 3) {
        w_carry[0] = wt[3][0];
        w_carry[1] = wt[3][1];
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  {
    float b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) fold_part(1, j, w_carry, b4);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      colred[(nsteps - 1) % 3][3 * 32 + h2 * 16 + c16][wave * 4 + g] = csA_carry[h2] + (b4[2 * h2] + b4[2 * h2 + 1]);
  }
  float* red = reinterpret_cast<float*>(lds_raw);
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 128 + 16 * rt + 4 * g + i) * RED + c16] = rsum[rt][i];
  __syncthreads();
  if (nsteps >= 2) flush(nsteps - 2);
  flush(nsteps - 1);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = tid + 256 * k, j = r0 + row;
    if (j < n) {
      float s = 0.f;
#pragma unroll
      for (int l = 0; l < 16; ++l) s += red[row * RED + l];
      const float w = wv[j];
      p.rs[head * p.cap + j] = s - (w > 0.f ? 1.0f / w : 0.f);
    }
  }
}

// Small caches: one work-group per pair of 128-key blocks (gram_pairs_unit).
__global__ __launch_bounds__(256) void k_gram_pairs(GramParams p) { gram_pairs_unit(p, blockIdx.x); }

// R and Z per key: own row sums plus the column sums of the blocks that
// computed this key's block as their column block, in slot order.  A thread
// takes V consecutive keys (one block, as V divides the block size) with
// V-wide loads of every slot; V = 4 needs cap % 4 == 0 for aligned rows.
template <int V>
__global__ __launch_bounds__(256) void k_gram_fin(GramParams p) {
  typedef float fv_t __attribute__((ext_vector_type(V)));
  __shared__ uint32_t lh[kHistBins];
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z, tid = threadIdx.x;
  const long head = (long)bi * p.hkv + h;
  const int j = (chunk * 256 + tid) * V;
  // Everything but the slots past the first batch is requested before the
  // length arrives: the key's weights, importance and own-block row sums and
  // its first slots, as many as a full cache gives the work-group's last
  // block (the count for n = cap; a shorter sequence needs at most as many;
  // uniform over the work-group, so the slot offsets stay scalar), clamped
  // to SB.
  const int jl = min(j, p.cap - V);
  const int nbc = (p.cap + p.bs - 1) / p.bs;
  const int Jw = min((chunk * 256 + 255) * V, p.cap - 1) / p.bs;
  const int ntc = p.pairs ? nbc : (nbc - 1) / 2 + (nbc % 2 == 0 && nbc >= 2 && Jw >= nbc / 2 ? 1 : 0);
  const float* pp = p.part + head * (long)p.nsmax * p.cap + jl;
  const long ol = head * p.cap + jl;
  auto ld = [](const float* q) { return *reinterpret_cast<const fv_t*>(q); };
  const fv_t w = ld(p.inv_norm + head * (long)p.wstride + jl);
  const fv_t imp = ld(p.i_in + ol);
  fv_t tot;
  if (p.pairs) {
#pragma unroll
    for (int e = 0; e < V; ++e) tot[e] = 0.f;
  } else {
    tot = ld(p.rs + ol);
  }
  constexpr int SB = 32;
  fv_t a[SB];
  if constexpr (V == 4) {
    // buffer loads: one per-lane offset, the slot row as a scalar offset (the
    // launcher keeps a head's slots below 2^31 bytes for this form)
    const auto pr = buf_rsrc(p.part + head * (long)p.nsmax * p.cap, (uint32_t)p.nsmax * p.cap * 4u);
#pragma unroll
    for (int u = 0; u < SB; ++u)
      a[u] = __builtin_bit_cast(fv_t, buf_ld128(pr, (uint32_t)jl * 4u, (uint32_t)min(u, max(ntc, 1) - 1) * p.cap * 4u));
  } else {
#pragma unroll
    for (int u = 0; u < SB; ++u) a[u] = ld(pp + (long)min(u, max(ntc, 1) - 1) * p.cap);
  }
  const int n = clamp_len(p.lengths[bi], p.cap);
  // pairs: one slot per block of the cache.  Otherwise slot s holds the
  // contribution of block J - (s+1) for s < (nb-1)/2, and the slot of
  // distance nb/2 (nb even, filled only for J >= nb/2) is the next one,
  // (nb-1)/2: either way the key's slots are a prefix, added in slot order.
  // The first batch is added before anything branches on n, which keeps its
  // loads ahead of the length's.
  const int nb = (n + p.bs - 1) / p.bs, J = jl / p.bs;
  const int nt = p.pairs ? nb : (nb - 1) / 2 + (nb % 2 == 0 && nb >= 2 && J >= nb / 2 ? 1 : 0);
#pragma unroll
  for (int u = 0; u < SB; ++u) {
    const bool in = u < nt;
#pragma unroll
    for (int e = 0; e < V; ++e) tot[e] += in ? a[u][e] : 0.f;
  }
  if (chunk * 256 * V >= n) return;
  if (p.hist)
    for (int t = tid; t < kHistBins; t += 256) lh[t] = 0u;
  __syncthreads();
  if (j < n) {
    // later batches (more than SB slots: caches beyond 32K keys); indices
    // past the last slot re-read it and add 0
    for (int s0 = SB; s0 < nt; s0 += SB) {
#pragma unroll
      for (int u = 0; u < SB; ++u) a[u] = ld(pp + (long)min(s0 + u, nt - 1) * p.cap);
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const bool in = s0 + u < nt;
#pragma unroll
        for (int e = 0; e < V; ++e) tot[e] += in ? a[u][e] : 0.f;
      }
    }
    const float inv_nm1 = n > 1 ? 1.0f / (float)(n - 1) : 0.f;
    fv_t red, z;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float t = tot[e];
      // pairs: the self term w_j ||k_j||^2 = 1 / w_j (0 for a zero key)
      if (p.pairs) t -= w[e] > 0.f ? 1.0f / w[e] : 0.f;
      red[e] = w[e] * t * inv_nm1;
      z[e] = fmaf(p.lambda, imp[e], -(1.0f - p.lambda) * red[e]);
    }
    const long o = head * p.cap + j;
    if (j + V <= n) {
      if (p.r_out) *reinterpret_cast<fv_t*>(p.r_out + o) = red;
      *reinterpret_cast<fv_t*>(p.z_out + o) = z;
    } else {
      for (int e = 0; e < V && j + e < n; ++e) {
        if (p.r_out) p.r_out[o + e] = red[e];
        p.z_out[o + e] = z[e];
      }
    }
    if (p.hist)
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (j + e < n) atomicAdd(&lh[hist_bin(score_key(z[e]))], 1u);
  }
  if (p.hist) {
    __syncthreads();
    for (int t = tid; t < kHistBins; t += 256)
      if (lh[t]) atomicAdd(&p.hist[head * kHistStride + t], lh[t]);
  }
}

template <typename E, int D>
static hipError_t gram_t(const GramParams& p, hipStream_t s, Trace* tr) {
  const int blocks = (p.cap + 255) / 256 * p.hkv * p.b;
  return launch_k(k_gram<E, D>, dim3(blocks), dim3(256), s, tr, p);
}

// bf16 keys of 128 dimensions use 512-key blocks once there are at least 16
// of them per head at full length (enough work-groups to fill the chip at the
// shapes this path serves); everything else uses 256-key blocks.
GramParams gram_config(int dt, int d, const GramParams& p_in) {
  GramParams p = p_in;
  const bool big = dt == 0 && d == 128 && p.cap >= 8192;
  const bool small = dt == 0 && d == 128 && p.cap <= kGramPairCap;
  p.bs = big ? 512 : (small ? 128 : 256);
  p.pairs = small ? 1 : 0;
  return p;
}

long gram_pair_units(const GramParams& p) {
  const long nbh = (p.cap + 127) / 128;
  return nbh * (nbh + 1) / 2 * p.hkv * p.b;
}

hipError_t launch_gram(int dt, int d, const GramParams& p_in, hipStream_t s, Trace* tr) {
  const GramParams p = gram_config(dt, d, p_in);
  // one-dimensional grids: every work-group index must fit an int
  const long nbk = (p.cap + p.bs - 1) / p.bs;
  if ((p.pairs ? gram_pair_units(p) : nbk * p.hkv * p.b) >= (1L << 31)) return hipErrorInvalidValue;
  hipError_t e;
  if (p.bs == 512) e = launch_k(k_gram512, dim3((p.cap + 511) / 512 * p.hkv * p.b), dim3(256), s, tr, p);
  else if (p.pairs) e = launch_k(k_gram_pairs, dim3(gram_pair_units(p)), dim3(256), s, tr, p);
  else if (dt == 0) e = d == 64 ? gram_t<BF16, 64>(p, s, tr) : gram_t<BF16, 128>(p, s, tr);
  else e = d == 64 ? gram_t<F32, 64>(p, s, tr) : gram_t<F32, 128>(p, s, tr);
  if (e != hipSuccess) return e;
  return launch_gram_fin(p, s, tr);
}

hipError_t launch_gram_fin(const GramParams& p, hipStream_t s, Trace* tr) {
  auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
  if (p.cap % 4 == 0 && (long)p.nsmax * p.cap * 4 < (1L << 31) && al16(p.part) && al16(p.rs) &&
      al16(p.inv_norm) && al16(p.i_in) && al16(p.z_out) && al16(p.r_out))
    return launch_k(k_gram_fin<4>, dim3((p.cap + 1023) / 1024, p.hkv, p.b), dim3(256), s, tr, p);
  return launch_k(k_gram_fin<1>, dim3((p.cap + 255) / 256, p.hkv, p.b), dim3(256), s, tr, p);
}

}  // namespace kvsel
