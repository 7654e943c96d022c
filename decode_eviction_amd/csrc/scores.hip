// Streaming score kernels: attention statistics, importance pooling and the
// key-sum form of redundancy.
//
// R-KV importance (QbitAI R-KV article, section "R-KV三步走", importance
// scoring from multi-head attention): for KV head h the g*w window rows of its
// GQA group attend over the n cached keys; I[j] is the mean of their softmax
// rows.  The softmax needs each row's global max and sum of exponentials, so
// K is streamed twice:
//   k_stats  per 256-token chunk: logits on the matrix cores, per-row chunk
//            max / sum-exp (key-sum mode: key norms and the chunk's sum of
//            unit keys); ReFreeKV mode also stores the scaled logits;
//   k_reduce per head: merges chunk partials (online-softmax merge) and the
//            unit-key sums (R-KV calls of at most kFuseReduceChunks chunks
//            per head skip it: k_pool merges them itself);
//   k_pool   per 256-token chunk: logits again, p = exp(s - max) / sum,
//            I[j] = mean over rows; Gram mode writes the key weights
//            1/||k_j||; key-sum mode adds
//            R[j] = (u_j.S - u_j.u_j) / (n-1),  S = sum_i u_i, u = k/||k||
//            and Z[j] = lambda I[j] - (1-lambda) R[j].
//
// Tiles: each 256-thread work-group covers 256 tokens; each wave takes two
// 32-token tiles.  k_stats forms C[token][row] so a lane owns one query row
// and reduces over tokens in registers; k_pool forms C[row][token] so a lane
// owns one token and reduces over rows in registers (plus one lane swap).
#include "common.hpp"
#include "gram_pairs.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace kvsel {

// Four waves per SIMD (every work-group of a 32K-token head resident at
// once) where the two key tiles leave room for it; fp32 keys of 128
// dimensions take 128 registers by themselves.
template <typename E, int D>
constexpr int kStatsWaves = E::kBytes == 2 || D == 64 ? 4 : 1;

// The ReFreeKV single-tile form (bf16, d = 128) fits five.
template <typename E, int D, int MT, int MODE>
constexpr int kStatsWavesFor = MODE == kModeCut && MT == 1 && E::kBytes == 2 && D == 128 ? 5 : kStatsWaves<E, D>;

template <typename E, int D, int MT, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kStatsWavesFor<E, D, MT, MODE>)))
void k_stats(ScoreParams p) {
  using G = Geo<E, D>;
  constexpr int NC = G::kNC;
  constexpr int LE = G::kLaneElems;
  constexpr int PC = E::kPerChunk;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;

  // per-call and per-head duties by grid position
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) {
    int f = 0;
    for (int i = 0; i < p.b; ++i) f |= len_bad(p.lengths[i], p.cap) ? 1 : 0;
    *p.err = f;
  }
  if (p.hist && blockIdx.x == 0)  // the later passes accumulate into it (selection state with it)
    for (int t = tid; t < kHistStride; t += 256)
      p.hist[((long)blockIdx.z * p.hkv + blockIdx.y) * kHistStride + t] = 0u;
  int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  if (p.b > 1 && p.b <= kActiveFirstMaxB && !active_chunk(p.lengths, p.b, p.hkv, p.cap, p.nchunk, bi, h, chunk))
    return;
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int c0 = chunk * kChunk;
  const long head = (long)bi * p.hkv + h;
  if (c0 >= n) return;
  const char* kb = p.k + head * (long)p.cap * G::kRowBytes;
  const char* qb = p.q + (((long)bi * p.hq + (long)h * p.g) * p.w + p.rows0) * G::kRowBytes;

  using QSt = QStage<E, D, MT>;
  __shared__ u32x4_t qs[QSt::kWords];
  Frag<NC> qf[QSt::kLds ? 1 : MT];
  if constexpr (QSt::kLds) {
    QSt::issue(qs, qb, p.m, tid);
  } else {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int r = 32 * t + l32;
      load_frag<E, D>(qf[t], qb, r, r < p.m, hf);
    }
  }
  const int tok0 = c0 + wave * 64;
  Frag<NC> kf[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tok = tok0 + 32 * tt + l32;
    load_frag<E, D>(kf[tt], kb, tok, tok < n, hf);
  }

  // key-sum mode: key norms and the chunk's unit-key sum (the Gram form's
  // norms are taken in k_pool, which reads K from the last-level cache)
  auto norms = [&]() {
    if constexpr (MODE == kModeKeysum) {
      float inv[2];
  #pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float ss = frag_sumsq<E, NC>(kf[tt]);
        ss += xor32(ss);
        inv[tt] = inv_norm_of(ss);
      }
      {
        // this chunk's sum of unit keys: per lane its two tokens, then a
        // reduce-scatter over the 32 lanes of the half, then across waves
        // (the first reduce-scatter step is taken as the values are formed, so
        // that only half of them are ever held)
        float v[LE / 2];
        {
          const bool up = (l32 & 16) != 0;
  #pragma unroll
          for (int i = 0; i < LE / 2; ++i) {
            const int j = i / PC, e = i % PC;
            const float lo = fmaf(inv[0], frag_elem<E>(kf[0].c[j], e), inv[1] * frag_elem<E>(kf[1].c[j], e));
            const float hi = fmaf(inv[0], frag_elem<E>(kf[0].c[j + NC / 2], e),
                             inv[1] * frag_elem<E>(kf[1].c[j + NC / 2], e));
            v[i] = (up ? hi : lo) + __shfl_xor(up ? lo : hi, 16, 64);
          }
        }
        scatter_down<LE / 2, 8, PC>(v, l32);
        constexpr int R = 32 / NC;  // lanes of a half still to be summed
        __shared__ float red[256 * PC];
        float* mine = red + (wave * 64 + lane) * PC;
  #pragma unroll
        for (int e = 0; e < PC; ++e) mine[e] = v[e];
        __syncthreads();
        if (tid < D) {
          const int ch = tid / PC, e = tid % PC, hfd = ch & 1, j = ch >> 1;
          float a = 0.f;
  #pragma unroll
          for (int wv = 0; wv < 4; ++wv)
  #pragma unroll
            for (int q = 0; q < R; ++q) a += red[(wv * 64 + hfd * 32 + j * R + q) * PC + e];
          p.spart[(head * p.nchunk + chunk) * D + tid] = a;
        }
      }
    }
  };

  // per-row max and sum of 2^(t - max), t = logit * log2(e) / sqrt(d).  The
  // last key a query row sees is n-1, or n - krows + r for row r of the last
  // krows rows (causal); only waves past the smallest such limit mask keys.
  const bool causal = MODE == kModeCut && p.krows > 1;
  const bool full = tok0 + 63 <= (causal ? n - p.krows : n - 1);
  const float sc2 = p.scale2;
  __shared__ float2 wst[4][MT * 32];
  // cut mode, one row tile: the chunk's logits of up to kLgRows rows, rows
  // padded by 4 words so that the 16-byte writes of different rows spread
  // over the banks
  constexpr int kLgRows = 8, kLgStride = kChunk + 4;
  __shared__ __attribute__((aligned(16))) float lgs[MODE == kModeCut && MT == 1 ? kLgRows * kLgStride : 4];
  // row tile t from its two accumulator tiles C[token][row] (lane: query row
  // 32t + l32, tokens tile_row(i, hf) of each key tile)
  auto row_tile = [&](int t, const f32x16_t (&a)[2]) {
    const int lim = causal ? n - p.krows + (p.rows0 + 32 * t + l32) % p.krows : n - 1;
    // token of slot (tt, i) is tok0 + 4 hf + 32 tt + 8 (i / 4) + i % 4: the
    // masks compare constants against one per-lane value
    const int rel = lim - (tok0 + 4 * hf);
    float m = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = full || 32 * tt + 8 * (i >> 2) + (i & 3) <= rel;
        m = ok ? fmaxf(m, a[tt][i]) : m;
      }
    m = fmaxf(m, xor32(m));
    const float m2 = m * sc2;  // sc2 > 0: the max of the scaled logits
    float s = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool ok = full || 32 * tt + 8 * (i >> 2) + (i & 3) <= rel;
          const float e = exp2_fast(fmaf(a[tt][i], sc2, -m2));
          s += ok ? e : 0.f;
        }
    }
    s += xor32(s);
    if (hf == 0) wst[wave][32 * t + l32] = make_float2(m2, s);

    if constexpr (MODE == kModeCut) {
      // logits of the m rows in base-2 units (-inf where a row does not see
      // the key), 4 consecutive tokens per store; none when k_pool forms the
      // energies from recomputed logits
      // chunk-major ([head][chunk][row][token]): a work-group's logits are
      // one contiguous block.  Up to kLgRows rows go through LDS and are
      // written out whole after the barrier (a lane here holds 4 consecutive
      // tokens of one row: direct stores are 32-byte pieces of many lines)
      const int row = 32 * t + l32;
      if (p.logits && row < p.m) {
        const bool staged = MT == 1 && p.m <= kLgRows;
        float* lrow = p.logits + ((head * p.nchunk + chunk) * p.m + row) * (long)kChunk;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int tr = wave * 64 + 32 * tt + 8 * q4 + 4 * hf;  // token within the chunk
            f32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = full || 32 * tt + 8 * q4 + e <= rel ? a[tt][4 * q4 + e] * sc2 : -INFINITY;
            if (staged) *reinterpret_cast<f32x4_t*>(&lgs[row * kLgStride + tr]) = v;
            else *reinterpret_cast<f32x4_t*>(lrow + tr) = v;
          }
      }
    }
  };

  if constexpr (QSt::kLds) {
    QSt::landed(qs, tid);
    __syncthreads();
    // one row tile at a time: two accumulator tiles live, the query chunks
    // re-read from LDS per tile
    auto mfma_rows = [&](int t, f32x16_t (&a)[2]) {
      a[0] = zero16();
      a[1] = zero16();
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const u32x4_t qc = QSt::chunk(qs, t, l32, hf, j);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) a[tt] = mfma_chunk<E>(kf[tt].c[j], qc, a[tt]);
      }
    };
    if constexpr (MT == 1) {
      // the key fragments die in norms(), before the tile is read back
      f32x16_t a[2];
      mfma_rows(0, a);
      norms();
      row_tile(0, a);
    } else {
      norms();
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        f32x16_t a[2];
        mfma_rows(t, a);
        row_tile(t, a);
        // keeps the next tile's products after this one's epilogue (two
        // tiles in flight would double the accumulator registers)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    f32x16_t acc[MT][2];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[t][tt] = mfma_tile<E, NC>(kf[tt], qf[t], zero16());
    norms();
#pragma unroll
    for (int t = 0; t < MT; ++t) row_tile(t, acc[t]);
  }
  __syncthreads();
  if (tid < MT * 32) {
    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) softmax_merge(m, s, wst[wv][tid].x, wst[wv][tid].y);
    p.cstat[(head * p.nchunk + chunk) * p.mp + tid] = make_float2(m, s);
  }
  if constexpr (MODE == kModeCut && MT == 1) {
    // the staged logits: m rows of 256 tokens, contiguous in global memory
    if (p.logits && p.m <= kLgRows) {
      float* blk = p.logits + (head * p.nchunk + chunk) * p.m * (long)kChunk;
      for (int i = 4 * tid; i < p.m * kChunk; i += 4 * 256) {
        const int r = i / kChunk, c = i % kChunk;
        *reinterpret_cast<f32x4_t*>(blk + i) = *reinterpret_cast<const f32x4_t*>(&lgs[r * kLgStride + c]);
      }
    }
  }
}

// One work-group of 1024 threads per head.  Chunk partials are spread over
// all threads with several independent loads in flight per thread, then
// merged through LDS in a fixed order (deterministic).
template <int D, int MODE>
__global__ __launch_bounds__(1024) void k_reduce(ScoreParams p) {
  constexpr int U = 4;
  __shared__ float2 part[1024];
  __shared__ float spar[1024];
  const int h = blockIdx.x, bi = blockIdx.y, tid = threadIdx.x;
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int nch = (n + kChunk - 1) / kChunk;
  const long head = (long)bi * p.hkv + h;
  {
    const int r = tid % p.mp, gi = tid / p.mp, G = 1024 / p.mp;
    float m = -INFINITY, s = 0.f;
    const float2* cs = p.cstat + head * p.nchunk * p.mp + r;
    for (int c0 = gi; c0 < nch; c0 += G * U) {
      float2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * G;
        v[u] = c < nch ? cs[(long)c * p.mp] : make_float2(-INFINITY, 0.f);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) softmax_merge(m, s, v[u].x, v[u].y);
    }
    part[tid] = make_float2(m, s);
  }
  if constexpr (MODE == kModeKeysum) {
    const int dim = tid % D, gi = tid / D, G = 1024 / D;
    const float* sp = p.spart + head * p.nchunk * D + dim;
    float a = 0.f;
    for (int c0 = gi; c0 < nch; c0 += G * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * G;
        v[u] = c < nch ? sp[(long)c * D] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) a += v[u];
    }
    spar[tid] = a;
  }
  __syncthreads();
  if (tid < p.mp) {
    float m = -INFINITY, s = 0.f;
    for (int g = 0; g < 1024 / p.mp; ++g) softmax_merge(m, s, part[g * p.mp + tid].x, part[g * p.mp + tid].y);
    p.rstat[head * p.mp + tid] = make_float2(m, s > 0.f ? 1.0f / s : 0.f);
  }
  if constexpr (MODE == kModeKeysum) {
    if (tid < D) {
      float a = 0.f;
      for (int g = 0; g < 1024 / D; ++g) a += spar[g * D + tid];
      p.ssum[head * D + tid] = a;
    }
  }
}

template <typename E, int D, int MT, int MODE>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(MT > 1 && MODE != kModeCut ? kStatsWaves<E, D> : 1)))
void k_pool(ScoreParams p) {
  using G = Geo<E, D>;
  constexpr int NC = G::kNC;
  constexpr int LE = G::kLaneElems;
  constexpr int PC = E::kPerChunk;
  int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  if (p.b > 1 && p.b <= kActiveFirstMaxB && !active_chunk(p.lengths, p.b, p.hkv, p.cap, p.nchunk, bi, h, chunk))
    return;
#include "pool_body.inc"
}

// Short Gram-form caches: the pooling units (importance and the key weights
// the finish uses) and the pair-block Gram units (which weigh keys from
// their own fragments) in one grid.  Both read only K and what k_stats
// wrote, so they are independent: the pooling work-groups come first (their
// count rounded up to a multiple of 8, so that the Gram units keep their
// XCD-major order) and fill CUs the pair units leave idle in their second
// round.  Used where the one-launch score units cannot run beside the pairs
// (k_scores_pairs in fused.hip) and with KVSEL_SEPARATE_KERNELS=1.
struct PoolPairsParams {
  ScoreParams s;
  GramParams g;
  int npool;  // pooling work-groups, a multiple of 8
};

__global__ __launch_bounds__(256) void k_pool_pairs(PoolPairsParams pp) {
  const int bx = blockIdx.x;
  if (bx >= pp.npool) {
    gram_pairs_unit(pp.g, bx - pp.npool);
    return;
  }
  using E = BF16;
  constexpr int D = 128, MT = 1, MODE = kModeGram;
  using G = Geo<E, D>;
  constexpr int NC = G::kNC;
  constexpr int LE = G::kLaneElems;
  constexpr int PC = E::kPerChunk;
  const ScoreParams& p = pp.s;
  if (bx >= p.nchunk * p.hkv * p.b) return;
  const int hb = bx / p.nchunk;
  int chunk = bx - hb * p.nchunk, h = hb % p.hkv, bi = hb / p.hkv;
  if (p.b > 1 && p.b <= kActiveFirstMaxB && !active_chunk_at(bx, p.lengths, p.b, p.hkv, p.cap, bi, h, chunk))
    return;
#include "pool_body.inc"
}


// ---------------------------------------------------------------- launchers

template <typename E, int D, int MT>
static hipError_t stats_t(int mode, const ScoreParams& p, hipStream_t s, Trace* tr) {
  const dim3 grid(p.nchunk, p.hkv, p.b);
  switch (mode) {
    case kModeGram: return launch_k(k_stats<E, D, MT, kModeGram>, grid, dim3(256), s, tr, p);
    case kModeKeysum: return launch_k(k_stats<E, D, MT, kModeKeysum>, grid, dim3(256), s, tr, p);
    default: return launch_k(k_stats<E, D, MT, kModeCut>, grid, dim3(256), s, tr, p);
  }
}

template <typename E, int D>
static hipError_t stats_d(int mode, const ScoreParams& p, hipStream_t s, Trace* tr) {
  switch (p.mp / 32) {
    case 1: return stats_t<E, D, 1>(mode, p, s, tr);
    case 2: return stats_t<E, D, 2>(mode, p, s, tr);
    case 4: return stats_t<E, D, 4>(mode, p, s, tr);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stats(int dt, int d, int mode, const ScoreParams& p, hipStream_t s, Trace* tr) {
  if (dt == 0) return d == 64 ? stats_d<BF16, 64>(mode, p, s, tr) : stats_d<BF16, 128>(mode, p, s, tr);
  return d == 64 ? stats_d<F32, 64>(mode, p, s, tr) : stats_d<F32, 128>(mode, p, s, tr);
}

hipError_t launch_reduce(int d, int mode, const ScoreParams& p, hipStream_t s, Trace* tr) {
  const dim3 grid(p.hkv, p.b);
  if (mode == kModeKeysum)
    return d == 64 ? launch_k(k_reduce<64, kModeKeysum>, grid, dim3(1024), s, tr, p)
                   : launch_k(k_reduce<128, kModeKeysum>, grid, dim3(1024), s, tr, p);
  return launch_k(k_reduce<128, kModeGram>, grid, dim3(1024), s, tr, p);
}

template <typename E, int D, int MT>
static hipError_t pool_t(int mode, const ScoreParams& p, hipStream_t s, Trace* tr) {
  const dim3 grid(p.nchunk, p.hkv, p.b);
  switch (mode) {
    case kModeKeysum: return launch_k(k_pool<E, D, MT, kModeKeysum>, grid, dim3(256), s, tr, p);
    case kModeCut: return launch_k(k_pool<E, D, MT, kModeCut>, grid, dim3(256), s, tr, p);
    default: return launch_k(k_pool<E, D, MT, kModeGram>, grid, dim3(256), s, tr, p);
  }
}

template <typename E, int D>
static hipError_t pool_d(int mode, const ScoreParams& p, hipStream_t s, Trace* tr) {
  switch (p.mp / 32) {
    case 1: return pool_t<E, D, 1>(mode, p, s, tr);
    case 2: return pool_t<E, D, 2>(mode, p, s, tr);
    case 4: return pool_t<E, D, 4>(mode, p, s, tr);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pool_pairs(const ScoreParams& p, const GramParams& g, hipStream_t s, Trace* tr) {
  const long npool = ((long)p.nchunk * p.hkv * p.b + 7) / 8 * 8;
  const long total = npool + gram_pair_units(g);
  if (total >= (1L << 31)) return hipErrorInvalidValue;
  const PoolPairsParams pp{p, g, (int)npool};
  return launch_k(k_pool_pairs, dim3((unsigned)total), dim3(256), s, tr, pp);
}

hipError_t launch_pool(int dt, int d, int mode, const ScoreParams& p, hipStream_t s, Trace* tr) {
  if (dt == 0) return d == 64 ? pool_d<BF16, 64>(mode, p, s, tr) : pool_d<BF16, 128>(mode, p, s, tr);
  return d == 64 ? pool_d<F32, 64>(mode, p, s, tr) : pool_d<F32, 128>(mode, p, s, tr);
}

}  // namespace kvsel
