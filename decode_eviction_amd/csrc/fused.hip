// One launch for the whole R-KV step on short caches (key-sum redundancy).
//
// R-KV compresses the cache while decoding (QbitAI R-KV article, section
// "R-KV三步走": importance from the window's attention, redundancy from key
// cosine similarity, joint eviction under a KV budget), so the step runs on
// a small cache very often: the decode loop scores a 2176-slot cache every
// 128 tokens.  There the separate passes (statistics, pooling, threshold,
// compaction) are each bound by launch and memory latency, not bandwidth.
// k_rkv_fused runs them in one grid, one 256-thread work-group per
// 256-token chunk and head, with two per-head barriers:
//   1. logits on the matrix cores, per-row chunk max / sum of 2^(t - max),
//      key norms and the chunk's sum of unit keys (as k_stats);  barrier A
//   2. every work-group merges its head's chunk partials in the same fixed
//      order, then importance, the key-sum redundancy and Z for its tokens
//      (as k_pool), and publishes its tokens' order-preserving score keys;
//      barrier B
//   3. every work-group loads the head's whole key row (at most 4096 keys)
//      into LDS and selects there: a 2048-bin histogram of the top 11 bits,
//      then rounds of 11 bits inside the bin that holds the B-th largest key,
//      give the threshold key and how many of its copies are kept (lowest
//      positions first); one scan over the row gives every kept position its
//      ascending output slot.  Each work-group writes the slots of its own
//      positions and copies those K rows (still in registers) and V rows
//      (prefetched into LDS at the start).
// The arithmetic of phases 1 and 2 is the one of k_stats / k_pool (same
// expressions, same merge order), so the scores equal the multi-kernel
// path's bit for bit, and the selection is exact.
//
// Barriers.  Values that cross work-groups are 64-bit words, the value in
// the low half and the call's tag in the high half, written and read with
// device-scope accesses (they pass between XCDs).  A work-group issues its
// words, then writes a flag word (the tag and the barrier's number) into its
// slot of the head's flag row; a reader waits until the row holds every
// flag, then reads the words and reads again any whose tag is not there yet
// (its store was issued before the flag's but may land later).
// The tag (head_tag) combines the head's epoch, a counter in the workspace
// that each call advances by one after barrier A, with the call's salt from
// the host, so neither what a fresh workspace holds nor what earlier calls
// left there passes for this call's.  No initialisation kernel is needed and graph
// replays work.  The host launches this kernel only when the whole grid fits
// on the device at once, so every wait ends; a wait that still exceeds its
// poll limit sets bit 2 of the error word and continues.
#include "common.hpp"
#include "gram_pairs.hpp"
#include "kernels.hpp"
#include "scan.hpp"
#include "tiles.hpp"

namespace kvsel {

constexpr int kFusedKeys = kFusedMaxChunks * kChunk;   // 4096

// The head's flag row of barrier `which` (A: 0, B: 1).
__device__ __forceinline__ uint64_t* flag_row(const FusedParams& p, int which, long head) {
  return p.flags + ((long)which * p.b * p.hkv + head) * kFusedMaxChunks;
}

// This work-group's signal, once every wave has issued its tagged words: the
// call's tag and the barrier's number in one word.
__device__ __forceinline__ void signal(const FusedParams& p, int which, long head, int chunk,
                                       uint32_t tag, int tid) {
  __syncthreads();
  if (tid == 0) st_dev(flag_row(p, which, head) + chunk, tagged(tag, (uint32_t)which + 1u));
}

// Wait (wave 0 polls) until the head's nwg work-groups have signalled.
__device__ __forceinline__ void wait_flags(const FusedParams& p, int which, long head, int nwg,
                                           uint32_t tag, int tid) {
  if (tid < kWave) {
    const uint64_t tok = tagged(tag, (uint32_t)which + 1u);
    const uint64_t* fl = flag_row(p, which, head);
    bool ok = false;
    for (int it = 0; it < kSpinLimit && !ok; ++it) {
      const uint64_t v = tid < nwg ? ld_dev(fl + tid) : tok;
      ok = __ballot(v != tok) == 0ull;
      if (!ok) __builtin_amdgcn_s_sleep(2);
    }
    if (!ok && tid == 0) atomicOr(p.err, 4);
  }
  __syncthreads();
}

// The value of a tagged word already read as w: read again while the tag is
// missing.
__device__ __forceinline__ uint32_t untag(const FusedParams& p, const uint64_t* at, uint64_t w,
                                          uint32_t tag) {
  for (int it = 0; (uint32_t)(w >> 32) != tag; ++it) {
    if (it == kSpinLimit) {
      atomicOr(p.err, 4);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    w = ld_dev(at);
  }
  return (uint32_t)w;
}

__device__ __forceinline__ int fused_budget(const FusedParams& p, int h) {
  if (!p.budgets) return p.budget;
  const int v = p.budgets[h];
  return v < 0 ? 0 : (v > p.budget ? p.budget : v);
}

// Phase 1 for one 256-token chunk, as k_stats computes it (one tile of up to
// 32 query rows); each wave holds two 32-token key tiles, tokens tok0 ..
// tok0 + 63.  Hands the chunk's partials to the sinks: stat(r, max, sum of
// 2^(t - max)) for the 32 rows and, with kSums (the key-sum form),
// sum(dim, s) for the D dimensions of the chunk's sum of unit keys.  sqs
// receives each lane's half-row squared norms (for the pooling phase).
template <typename E, int D, bool kSums, typename StatSink, typename SumSink>
__device__ __forceinline__ void chunk_partials(const Frag<Geo<E, D>::kNC> (&kf)[2], const u32x4_t* qs,
                                               int n, int tok0, float sc2, float (&sqs)[2],
                                               float2 (*wst)[32], float* red, int tid,
                                               StatSink&& stat, SumSink&& sum) {
  using G = Geo<E, D>;
  using QSt = QStage<E, D, 1>;
  constexpr int NC = G::kNC, LE = G::kLaneElems, PC = E::kPerChunk, NW = 4;
  const int wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // the row statistics first, so that the accumulator tiles are dead before
  // the unit-key values are formed (the keys stay live for the pooling)
  {
    f32x16_t a[2];
    a[0] = zero16();
    a[1] = zero16();
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const u32x4_t qc = QSt::chunk(qs, 0, l32, hf, j);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) a[tt] = mfma_chunk<E>(kf[tt].c[j], qc, a[tt]);
    }
    const bool full = tok0 + 63 <= n - 1;
    const int rel = n - 1 - (tok0 + 4 * hf);
    float m = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = full || 32 * tt + 8 * (i >> 2) + (i & 3) <= rel;
        m = ok ? fmaxf(m, a[tt][i]) : m;
      }
    m = fmaxf(m, xor32(m));
    const float m2 = m * sc2;
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
    if (hf == 0) wst[wave][l32] = make_float2(m2, s);
  }
  if constexpr (!kSums) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) sqs[tt] = frag_sumsq<E, NC>(kf[tt]);
    __syncthreads();
  } else {
    float inv[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sqs[tt] = frag_sumsq<E, NC>(kf[tt]);
      float ss = sqs[tt];
      ss += xor32(ss);
      inv[tt] = inv_norm_of(ss);
    }
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
    float* mine = red + (wave * 64 + lane) * PC;
#pragma unroll
    for (int e = 0; e < PC; ++e) mine[e] = v[e];
    __syncthreads();
    if (tid < D) {
      constexpr int R = 32 / NC;
      const int ch = tid / PC, e = tid % PC, hfd = ch & 1, j = ch >> 1;
      float s = 0.f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv)
#pragma unroll
        for (int q = 0; q < R; ++q) s += red[(wv * 64 + hfd * 32 + j * R + q) * PC + e];
      sum(tid, s);
    }
  }
  if (tid < 32) {
    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) softmax_merge(m, s, wst[wv][tid].x, wst[wv][tid].y);
    stat(tid, m, s);
  }
}

// The attention that token l32 of key tile kf receives from the window's
// rows, summed (the importance before its 1/m), as k_pool computes it from
// the merged row statistics rs (max, 1/sum; zero for rows past m) in LDS.
// Both lanes of the token (hf = 0, 1) return the same value.
template <typename E, int D>
__device__ __forceinline__ float token_attention(const Frag<Geo<E, D>::kNC>& kf, const u32x4_t* qs,
                                                 const float2* rs, float sc2, int l32, int hf) {
  using QSt = QStage<E, D, 1>;
  constexpr int NC = Geo<E, D>::kNC;
  // at most two query chunks and four row records read ahead from LDS (the
  // keys stay in registers: the one-launch score pass runs at four waves
  // per SIMD)
  f32x16_t c = zero16();
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    c = mfma_chunk<E>(QSt::chunk(qs, 0, l32, hf, j), kf.c[j], c);
    if (j % 2 == 1) asm volatile("" ::: "memory");
  }
  float isum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float2 st = rs[tile_row(i, hf)];
    isum = fmaf(exp2_fast(fmaf(c[i], sc2, -st.x)), st.y, isum);
    if (i % 4 == 3) asm volatile("" : "+v"(isum)::"memory");
  }
  isum += xor32(isum);
  return isum;
}

// Phase 2 for a wave's two key tiles, as k_pool computes it: importance, the
// key-sum redundancy and Z of tokens tok0 + 32 tt + l32 from the merged row
// statistics rs (max, 1/sum; zero for rows past m) and the head's sum of
// unit keys ssh, both in LDS.  Both lanes of a token (hf = 0, 1) return the
// same values.
template <typename E, int D>
__device__ __forceinline__ void pool_tokens(const Frag<Geo<E, D>::kNC> (&kf)[2], const u32x4_t* qs,
                                            const float2* rs, const float* ssh,
                                            const float (&sqs)[2], int n, int m, float sc2,
                                            float lambda, int tid, float (&imp)[2], float (&rd)[2],
                                            float (&z)[2]) {
  constexpr int NC = Geo<E, D>::kNC, PC = E::kPerChunk;
  // LDS addresses recomputed here rather than kept from the partials
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  float dots[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int q = 0; q < PC / 4; ++q) {
      const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(&ssh[frag_dim<E>(j, 4 * q, hf)]);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dots[tt] = fmaf(frag_elem<E>(kf[tt].c[j], 4 * q + e), s4[e], dots[tt]);
      if ((j * (PC / 4) + q) % 4 == 3) asm volatile("" : "+v"(dots[0]), "+v"(dots[1])::"memory");
    }
  const float inv_m = 1.0f / (float)m;
  const float inv_nm1 = n > 1 ? 1.0f / (float)(n - 1) : 0.f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    imp[tt] = token_attention<E, D>(kf[tt], qs, rs, sc2, l32, hf) * inv_m;
    float ss = sqs[tt];
    ss += xor32(ss);
    const float inv = inv_norm_of(ss);
    float dot = dots[tt];
    dot += xor32(dot);
    rd[tt] = fmaf(inv, dot, -(inv * inv) * ss) * inv_nm1;
    z[tt] = fmaf(lambda, imp[tt], -(1.0f - lambda) * rd[tt]);
    __builtin_amdgcn_sched_barrier(0);  // one accumulator tile live at a time
  }
}

// The need-th largest (need >= 1, at most the count of keys in play) of the
// keys v[i] that bit i of `play` marks, over the work-group's threads, by
// rounds of 11-bit histograms in lh (2048 counters) until one key value is
// left: returns that key and how many of its copies rank within the first
// need.  The slot-reuse step's split of threshold ties by position.
template <int KPT, int NW>
__device__ __noinline__ uint2 nth_largest(const uint32_t (&v)[KPT], uint32_t play, uint32_t need,
                                          uint32_t* lh, uint32_t* wsum, uint32_t* bc, int tid) {
  uint32_t lo = 0u, hi = 0xffffffffu;
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > kHistBits ? bits - kHistBits : 0;
    const int nb = (int)(span >> shift) + 1;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) lh[8 * tid + i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t off = v[i] - lo;
      if (((play >> i) & 1u) && off <= span) atomicAdd(&lh[off >> shift], 1u);
    }
    __syncthreads();
    uint32_t rb[8], rs = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rb[i] = 8 * tid + i < nb ? lh[8 * tid + i] : 0u;
      rs += rb[i];
    }
    const uint2 sc = block_scan_u32<NW>(rs, wsum, tid);
    uint32_t above = sc.y - sc.x - rs;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above < need && above + rb[i] >= need) {
        bc[0] = 8 * tid + i;
        bc[1] = above;
      }
      above += rb[i];
    }
    __syncthreads();
    const uint32_t bin = bc[0];
    need -= bc[1];
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)bin << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
  }
  return make_uint2(lo, need);
}

// SLOTS: the slot-reuse form (kvsel_score_evict_slots): the same scores and
// threshold, ties at the threshold kept by lower token position (the
// caller's position map; equal positions: lower slot), and instead of the
// compaction the evicted slots listed in slot order; V is not read.
// GRAM (with SLOTS): the Gram form's finish instead of phases 1 and 2: Z of
// each token from the pooling's importance, the key weights and the
// pair-block Gram slots (k_gram_fin's arithmetic, one token per thread),
// then phase 3 and the evicted list; neither q, K nor V is read.
template <typename E, int D, bool SLOTS, bool GRAM>
__global__ __launch_bounds__(256) void k_rkv_fused(FusedParams p) {
  static_assert(SLOTS || !GRAM, "the Gram finish serves the slot-reuse form");
  using G = Geo<E, D>;
  constexpr int NC = G::kNC;
  constexpr int LE = G::kLaneElems;
  constexpr int PC = E::kPerChunk;
  constexpr int RB = G::kRowBytes;
  constexpr int NW = 4;
  constexpr int KPT = kFusedKeys / 256;  // keys of the row per thread in phase 3
  static_assert(RB * kChunk <= 64 * 1024, "V chunk staged in LDS");
  static_assert(D <= 128, "unit-key sums fit the partial record");
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const long head = (long)bi * p.hkv + h;
  const int c0 = chunk * kChunk;

  if (chunk == 0 && h == 0 && bi == 0 && tid == 0) {
    int f = 0;
    for (int i = 0; i < p.b; ++i) f |= len_bad(p.lengths[i], p.cap) ? 1 : 0;
    if (p.budgets)
      for (int i = 0; i < p.hkv; ++i) f |= (p.budgets[i] < 0 || p.budgets[i] > p.budget) ? 2 : 0;
    // device scope, as the other work-groups' atomicOr of bit 2: a plain
    // store would stay in this XCD's L2 and, written back at the end,
    // could overwrite a bit set meanwhile from another XCD
    __hip_atomic_store(p.err, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int B = fused_budget(p, h);
  int32_t* out = SLOTS ? p.evict + head * (long)p.evict_stride : p.idx + head * p.budget;
  if constexpr (SLOTS) {
    // n - min(B, n) evicted slots, then -1
    const int nev = n - min(n, B);
    if (chunk == 0) {
      for (int t = nev + tid; t < p.evict_stride; t += 256) out[t] = -1;
      if (tid == 0) p.n_evict[head] = nev;
    }
  } else if (chunk == 0) {
    for (int t = min(n, B) + tid; t < p.budget; t += 256) out[t] = -1;
  }
  if (c0 >= n) return;
  const int nwg = (n + kChunk - 1) / kChunk;
  const uint64_t ep = ld_dev(p.epoch + head);
  const uint32_t tag = head_tag(ep, head, p.salt);
  const char* kb = p.k + head * (long)p.cap * RB;
  const char* qb = p.q + ((long)bi * p.hq + (long)h * p.g) * p.w * RB;
  uint64_t* pa = p.pub_a + head * kFusedMaxChunks * kFusedWordsA;

  // q, then the chunk's keys (through a buffer resource that ends at token n:
  // keys past it read as zeros, as load_frag gives them, without a branch),
  // then V, which only the copies at the end need
  using QSt = QStage<E, D, 1>;
  __shared__ u32x4_t qs[QSt::kWords];
  if constexpr (!GRAM) QSt::issue(qs, qb, p.m, tid);
  const int tok0 = c0 + wave * 64;
  Frag<NC> kf[2];
  if constexpr (!GRAM) {
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kb + (long)c0 * RB, (uint32_t)min(n - c0, kChunk) * RB);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t off = (uint32_t)((wave * 64 + 32 * tt + l32) * RB + hf * 16);
#pragma unroll
      for (int j = 0; j < NC; ++j) kf[tt].c[j] = buf_ld128(rk, off + 32 * j, 0);
    }
  }
  // V rows of the chunk into LDS (rows past cap arrive as zeros), for the
  // gather at the end
  __shared__ __attribute__((aligned(16))) char vl[kChunk * RB];
  if constexpr (!SLOTS) {
    const __amdgpu_buffer_rsrc_t rv =
        buf_rsrc(p.v + (head * p.cap + c0) * (long)RB, (uint32_t)(p.cap - c0) * RB);
    constexpr int PER_WAVE = kChunk * RB / (NW * 1024);
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int off = (wave * PER_WAVE + u) * 1024;
      buf_lds16(rv, vl + off, (uint32_t)(off + 16 * lane));
    }
  }

  uint64_t* pb = p.pub_b + head * p.cap;
  if constexpr (GRAM) {
    // Z of token c0 + tid as k_gram_fin forms it: the key's Gram slots (one
    // per 128-key block of the cache) added in slot order, less the self
    // term 1 / w_j, times w_j / (n - 1), then lambda I - (1 - lambda) R
    const int tz = c0 + tid;
    if (tz < n) {
      const int nt = (n + 127) / 128;
      const float* sp = p.gpart + head * (long)p.nsmax * p.cap + tz;
      const float w = p.inv_norm[head * (long)p.wstride + tz];
      const float imp = p.i_in[head * p.cap + tz];
      float tot = 0.f;
      for (int sl = 0; sl < nt; ++sl) tot += sp[(long)sl * p.cap];
      const float inv_nm1 = n > 1 ? 1.0f / (float)(n - 1) : 0.f;
      const float t = tot - (w > 0.f ? 1.0f / w : 0.f);
      const float red = w * t * inv_nm1;
      const float z = fmaf(p.lambda, imp, -(1.0f - p.lambda) * red);
      p.z_out[head * p.cap + tz] = z;
      if (n > B && B > 0) st_dev(pb + tz, tagged(tag, score_key(z)));
    }
  } else {
    // ---- phase 1: chunk statistics and unit-key sums (k_stats' arithmetic)
    const float sc2 = p.scale2;
    __shared__ float2 wst[NW][32];
    __shared__ float red[256 * PC];
    QSt::landed(qs, tid);
    __syncthreads();
    float sqs[2];
    uint64_t* rec = pa + chunk * kFusedWordsA;
    chunk_partials<E, D, true>(
        kf, qs, n, tok0, sc2, sqs, wst, red, tid,
        [&](int r, float m, float s) {
          st_dev(rec + 2 * r, tagged(tag, __float_as_uint(m)));
          st_dev(rec + 2 * r + 1, tagged(tag, __float_as_uint(s)));
        },
        [&](int dim, float s) { st_dev(rec + 64 + dim, tagged(tag, __float_as_uint(s))); });
    signal(p, 0, head, chunk, tag, tid);
    wait_flags(p, 0, head, nwg, tag, tid);
    if (chunk == 0 && tid == 0) st_dev(p.epoch + head, ep + 1);  // every work-group has read ep

    // ---- phase 2: merged statistics, importance, redundancy, Z (k_pool's arithmetic)
    __shared__ float2 rs[32];
    __shared__ __attribute__((aligned(16))) float ssh[D];
    if (tid < 32) {
      uint64_t cw[2 * kFusedMaxChunks];
  #pragma unroll
      for (int u = 0; u < kFusedMaxChunks; ++u) {
        const uint64_t* at = pa + min(u, nwg - 1) * kFusedWordsA + 2 * tid;
        cw[2 * u] = ld_dev(at);
        cw[2 * u + 1] = ld_dev(at + 1);
      }
      float m = -INFINITY, s = 0.f;
  #pragma unroll
      for (int u = 0; u < kFusedMaxChunks; ++u)
        if (u < nwg) {
          const uint64_t* at = pa + u * kFusedWordsA + 2 * tid;
          const float cm = __uint_as_float(untag(p, at, cw[2 * u], tag));
          const float cs = __uint_as_float(untag(p, at + 1, cw[2 * u + 1], tag));
          softmax_merge(m, s, cm, cs);
        }
      const float2 v = make_float2(m, s > 0.f ? 1.0f / s : 0.f);
      rs[tid] = tid < p.m ? v : make_float2(0.f, 0.f);
    }
    if (tid < D) {
      // the order k_pool merges them in: group g of 1024 / D takes chunks g,
      // g + 1024 / D, ...; the groups are added in turn
      constexpr int GD = 1024 / D, F = kFusedMaxChunks;
      uint64_t cw[F];
  #pragma unroll
      for (int u = 0; u < F; ++u) cw[u] = ld_dev(pa + min(u, nwg - 1) * kFusedWordsA + 64 + tid);
      float c[F];
  #pragma unroll
      for (int u = 0; u < F; ++u)
        c[u] = u < nwg ? __uint_as_float(untag(p, pa + u * kFusedWordsA + 64 + tid, cw[u], tag)) : 0.f;
      float s = 0.f;
  #pragma unroll
      for (int g = 0; g < GD; ++g) {
        float ag = 0.f;
  #pragma unroll
        for (int ci = g; ci < F; ci += GD) ag += ci < nwg ? c[ci] : 0.f;
        s += ag;
      }
      ssh[tid] = s;
    }
    __syncthreads();
    float imp[2], rd[2], z[2];
    pool_tokens<E, D>(kf, qs, rs, ssh, sqs, n, p.m, sc2, p.lambda, tid, imp, rd, z);
  #pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tok = tok0 + 32 * tt + l32;
      if (hf == 0 && tok < n) {
        p.z_out[head * p.cap + tok] = z[tt];
        if (n > B && B > 0) st_dev(pb + tok, tagged(tag, score_key(z[tt])));
      }
    }
  }

  // ---- output slots of this chunk's tokens (-1: evicted), then the copies
  __shared__ int32_t sl[kChunk];
  auto gather = [&]() {
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int lt = wave * 64 + 32 * tt + l32;
      const int slot = sl[lt];
      if (slot >= 0) {
        char* ko = p.k_out + (head * p.cap_out + slot) * (long)RB;
        char* vo = p.v_out + (head * p.cap_out + slot) * (long)RB;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          const int off = (2 * j + hf) * 16;
          *reinterpret_cast<u32x4_t*>(ko + off) = kf[tt].c[j];
          *reinterpret_cast<u32x4_t*>(vo + off) = *reinterpret_cast<const u32x4_t*>(vl + lt * RB + off);
        }
      }
    }
  };
  if constexpr (SLOTS) {
    if (B == 0 || n <= B) {  // every slot evicted (in slot order), or none
      if (B == 0 && c0 + tid < n) out[c0 + tid] = c0 + tid;
      return;
    }
  }
  if (B == 0) return;
  if (n <= B) {  // everything is kept, in place
    const int pos = c0 + tid;
    sl[tid] = pos < n ? pos : -1;
    if (pos < n) out[pos] = pos;
    gather();
    return;
  }
  signal(p, 1, head, chunk, tag, tid);
  wait_flags(p, 1, head, nwg, tag, tid);
  if constexpr (GRAM)  // no barrier A: every work-group has read ep by now
    if (chunk == 0 && tid == 0) st_dev(p.epoch + head, ep + 1);

  // ---- phase 3: the head's keys in LDS, the threshold, slots of this chunk
  __shared__ uint32_t kall[kFusedKeys];
  __shared__ uint32_t lh[kHistBins];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t bc[4];
  {
    uint64_t kw[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) kw[i] = ld_dev(pb + min(tid + 256 * i, n - 1));
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int pos = tid + 256 * i;
      if (pos < n) kall[pos] = untag(p, pb + pos, kw[i], tag);
    }
  }
  for (int t = tid; t < kHistBins; t += 256) lh[t] = 0u;
  __syncthreads();
  // thread t owns positions KPT t .. KPT t + KPT - 1 from here on
  uint32_t mk[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int pos = KPT * tid + i;
    mk[i] = pos < n ? kall[pos] : 0u;
    if (pos < n) atomicAdd(&lh[hist_bin(mk[i])], 1u);
  }
  __syncthreads();
  // level 1: the bin where the count from the top reaches B
  uint32_t hb[8], hs = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hb[i] = lh[8 * tid + i];
    hs += hb[i];
  }
  if (tid == 0) bc[0] = bc[1] = bc[2] = 0u;
  {
    const uint2 sc = block_scan_u32<NW>(hs, wsum, tid);
    uint32_t above = sc.y - sc.x - hs;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above < (uint32_t)B && above + hb[i] >= (uint32_t)B) {
        bc[0] = 8 * tid + i;
        bc[1] = above;
        bc[2] = hb[i];
      }
      above += hb[i];
    }
    __syncthreads();
  }
  uint32_t lo = bc[0] << (32 - kHistBits);
  uint32_t hi = lo | ((1u << (32 - kHistBits)) - 1u);
  uint32_t need = (uint32_t)B - bc[1];
  // rounds of 11 bits inside the bin (lh reused: thread t holds sub-bins
  // 8t .. 8t + 7) until one key value remains: the bin's 21 low bits take
  // at most two
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > kHistBits ? bits - kHistBits : 0;
    const int nb = (int)(span >> shift) + 1;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) lh[8 * tid + i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t off = mk[i] - lo;
      if (KPT * tid + i < n && off <= span) atomicAdd(&lh[off >> shift], 1u);
    }
    __syncthreads();
    uint32_t rb[8], rs = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rb[i] = 8 * tid + i < nb ? lh[8 * tid + i] : 0u;
      rs += rb[i];
    }
    const uint2 sc = block_scan_u32<NW>(rs, wsum, tid);
    uint32_t above = sc.y - sc.x - rs;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above < need && above + rb[i] >= need) {
        bc[0] = 8 * tid + i;
        bc[1] = above;
        bc[2] = rb[i];
      }
      above += rb[i];
    }
    __syncthreads();
    const uint32_t bin = bc[0];
    need -= bc[1];
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)bin << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
  }
  const uint32_t kth = lo, need_eq = need;  // keys above kth all kept; need_eq copies of kth
  {
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool ok = KPT * tid + i < n;
      cg += (ok && mk[i] > kth) ? 1u : 0u;
      ce += (ok && mk[i] == kth) ? 1u : 0u;
    }
    const uint2 sc = block_scan_u32<NW>(cg | (ce << 16), wsum, tid);
    // a consistent threshold keeps exactly B keys, so every slot below is in
    // [0, B); anything else (never seen) is flagged and nothing is written
    if ((sc.y & 0xffffu) + min(sc.y >> 16, need_eq) != (uint32_t)B) {
      if (tid == 0) atomicOr(p.err, 8);
      return;
    }
    if constexpr (SLOTS) {
      // kept: above the threshold, or one of the need_eq copies of it that
      // come first by (position, slot)
      uint32_t kept = 0u, tied = 0u;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool ok = KPT * tid + i < n;
        kept |= (ok && mk[i] > kth) ? 1u << i : 0u;
        tied |= (ok && mk[i] == kth) ? 1u << i : 0u;
      }
      if (need_eq == (sc.y >> 16) || !p.pos) {
        // every copy kept, or positions are the slots: the first need_eq
        // copies in slot order
        uint32_t eqb = sc.x >> 16;
#pragma unroll
        for (int i = 0; i < KPT; ++i)
          if ((tied >> i) & 1u) {
            kept |= eqb < need_eq ? 1u << i : 0u;
            ++eqb;
          }
      } else {
        // the copies split by position: the need_eq-th smallest position
        // among them (as the need_eq-th largest of ~pos), equal positions
        // in slot order
        const int32_t* pm = p.pos + head * (long)p.cap;
        uint32_t v2[KPT];
#pragma unroll
        for (int i = 0; i < KPT; ++i) v2[i] = ((tied >> i) & 1u) ? ~(uint32_t)pm[KPT * tid + i] : 0u;
        const uint2 pt = nth_largest<KPT, NW>(v2, tied, need_eq, lh, wsum, bc, tid);
        uint32_t c2 = 0;
#pragma unroll
        for (int i = 0; i < KPT; ++i) c2 += (((tied >> i) & 1u) && v2[i] == pt.x) ? 1u : 0u;
        uint32_t e2 = block_scan_u32<NW>(c2, wsum, tid).x;
#pragma unroll
        for (int i = 0; i < KPT; ++i)
          if ((tied >> i) & 1u) {
            if (v2[i] > pt.x) {
              kept |= 1u << i;
            } else if (v2[i] == pt.x) {
              kept |= e2 < pt.y ? 1u << i : 0u;
              ++e2;
            }
          }
      }
      // evicted slots in slot order: this thread's evicted positions follow
      // those of the threads before it
      uint32_t ne = 0;
#pragma unroll
      for (int i = 0; i < KPT; ++i) ne += (KPT * tid + i < n && !((kept >> i) & 1u)) ? 1u : 0u;
      uint32_t eb = block_scan_u32<NW>(ne, wsum, tid).x;
      const bool mine = KPT * tid >= c0 && KPT * tid < c0 + kChunk;
      const uint32_t nev = (uint32_t)(n - B);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int pos = KPT * tid + i;
        if (pos < n && !((kept >> i) & 1u)) {
          if (mine && eb < nev) out[eb] = pos;
          ++eb;
        }
      }
      return;
    }
    uint32_t gtb = sc.x & 0xffffu, eqb = sc.x >> 16;
    // this chunk's positions are owned by threads c0 / KPT .. (c0 + kChunk) / KPT - 1
    const bool mine = KPT * tid >= c0 && KPT * tid < c0 + kChunk;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int pos = KPT * tid + i;
      const bool ok = pos < n;
      int slot = -1;
      if (ok && mk[i] > kth) {
        slot = (int)(gtb + min(eqb, need_eq));
        ++gtb;
      } else if (ok && mk[i] == kth) {
        if (eqb < need_eq) slot = (int)(gtb + eqb);
        ++eqb;
      }
      if (mine) {
        sl[pos - c0] = slot;
        if (slot >= 0) out[slot] = pos;
      }
    }
  }
  gather();
}

hipError_t launch_fused(const FusedParams& p, hipStream_t s, Trace* tr) {
  const dim3 grid((p.cap + kChunk - 1) / kChunk, p.hkv, p.b);
  if (p.gpart) {  // the Gram finish serves the slot-reuse form
    if (!p.evict) return hipErrorInvalidValue;
    return launch_k(k_rkv_fused<BF16, 128, true, true>, grid, dim3(256), s, tr, p);
  }
  if (p.evict) return launch_k(k_rkv_fused<BF16, 128, true, false>, grid, dim3(256), s, tr, p);
  return launch_k(k_rkv_fused<BF16, 128, false, false>, grid, dim3(256), s, tr, p);
}

// ------------------------------------------------------------------------
// One-launch score pass (key-sum form on long caches; the importance and
// key weights of the Gram form on any cache).
//
// The multi-kernel pass streams K twice (k_stats, then k_pool after
// k_reduce, or k_pool merging the partials itself on short caches).
// k_scores_fused reads each key once: a work-group per 256-token chunk and
// head computes the chunk's partials as k_stats does and keeps its keys in
// registers; the head's first work-groups each merge one slice of the
// partials in k_reduce's order (the row statistics of rows 0-15 and 16-31,
// then, in the key-sum form, the unit-key sums 32 dimensions at a time);
// every work-group then pools its own tokens from the merged record as
// k_pool does: importance, redundancy, Z and the histogram in the key-sum
// form; importance and the inverse key norms 1/||k_j|| (the weights of the
// Gram kernels, which run next) in the Gram form.  The results equal the
// multi-kernel pass's bit for bit.
//
// Records that cross work-groups are tagged words (value in the low half,
// the call's tag for the head in the high half) written and read with
// device-scope accesses; a reader polls each word until it holds the tag, so
// arrival needs no separate flag and no store acknowledgement.  The merger
// of rows 0-15 advances the head's epoch once it has read every chunk's
// words (then every work-group of the head has read the epoch).  The host
// launches the kernel only when the whole grid fits on the device at once; a
// poll that still exceeds its limit sets bit 2 of the error word.

// One (chunk, head, sequence) unit of the score pass; k_scores_fused runs
// the units of a call in rounds (below).
template <typename E, int D, int MODE>
__device__ __forceinline__ void scores_fused_unit(const ScoresFusedParams& fp, int chunk, int h, int bi) {
  const ScoreParams& p = fp.s;
  using G = Geo<E, D>;
  using QSt = QStage<E, D, 1>;
  constexpr bool kGram = MODE == kModeGram;
  static_assert(kGram || MODE == kModeKeysum, "R-KV score forms");
  constexpr int NC = G::kNC, RB = G::kRowBytes, PC = E::kPerChunk;
  constexpr int W = kGram ? kGramWordsA : kFusedWordsA;
  // merge slices: rows 0-15, rows 16-31, then 32 dimensions each
  constexpr int NP = kGram ? 2 : 2 + D / 32;
  static_assert(D == 128 && (kGram || NP == kScoreMergeParts), "merge slices of the 128-dimension record");
  // the wave index in a scalar register (the compiler cannot prove tid >> 6
  // uniform): wave-derived offsets then take no vector registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const long head = (long)bi * p.hkv + h;
  const int c0 = chunk * kChunk;
  if (chunk == 0 && h == 0 && bi == 0 && tid == 0) {
    int f = 0;
    for (int i = 0; i < p.b; ++i) f |= len_bad(p.lengths[i], p.cap) ? 1 : 0;
    // device scope, as the other work-groups' atomicOr of bit 2: a plain
    // store would stay in this XCD's L2 and, written back at the end,
    // could overwrite a bit set meanwhile from another XCD
    __hip_atomic_store(p.err, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the head's first-level histogram (and the selection state after it)
  // starts at zero: chunk 0 clears it before it publishes its merged rows,
  // which every work-group reads before adding to it
  uint32_t* hg = p.hist ? p.hist + head * kHistStride : nullptr;
  if (hg && chunk == 0)
    for (int t = tid; t < kHistStride; t += 256) st_dev(hg + t, 0u);
  const int n = clamp_len(p.lengths[bi], p.cap);
  if (c0 >= n) return;
  const int nwg = (n + kChunk - 1) / kChunk;
  const uint64_t ep = ld_dev(fp.epoch + head);
  const uint32_t tag = head_tag(ep, head, fp.salt);
  const char* kb = p.k + head * (long)p.cap * RB;
  const char* qb = p.q + ((long)bi * p.hq + (long)h * p.g) * p.w * RB;

  __shared__ u32x4_t qs[QSt::kWords];
  QSt::issue(qs, qb, p.m, tid);
  const int tok0 = c0 + wave * 64;
  // the chunk's keys through a buffer resource that ends at token n: keys
  // past it read as zeros (as load_frag gives them), without a branch
  Frag<NC> kf[2];
  {
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kb + (long)c0 * RB, (uint32_t)min(n - c0, kChunk) * RB);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t off = (uint32_t)((wave * 64 + 32 * tt + l32) * RB + hf * 16);
#pragma unroll
      for (int j = 0; j < NC; ++j) kf[tt].c[j] = buf_ld128(rk, off + 32 * j, 0);
    }
  }
  __shared__ uint32_t lh[kGram ? 1 : kHistBins];
  if constexpr (!kGram)
    if (hg)
      for (int t = tid; t < kHistBins; t += 256) lh[t] = 0u;

  // ---- chunk partials (k_stats' arithmetic) as tagged words
  const float sc2 = p.scale2;
  __shared__ float2 wst[4][32];
  __shared__ float red[256 * PC];  // also the merge's group partials
  static_assert(256 * PC >= 2 * 32 * 16, "group partials of 16 rows fit");
  QSt::landed(qs, tid);
  __syncthreads();
  float sqs[2];
  uint64_t* pr = fp.part + head * p.nchunk * W;  // [chunk][W]
  uint64_t* mr = fp.merged + head * W;
  {
    uint64_t* rec = pr + (long)chunk * W;
    chunk_partials<E, D, !kGram>(
        kf, qs, n, tok0, sc2, sqs, wst, red, tid,
        [&](int r, float m, float s) {
          st_dev(rec + 2 * r, tagged(tag, __float_as_uint(m)));
          st_dev(rec + 2 * r + 1, tagged(tag, __float_as_uint(s)));
        },
        [&](int dim, float s) { st_dev(rec + 64 + dim, tagged(tag, __float_as_uint(s))); });
  }
  if constexpr (kGram) {
    // the weight 1/||k_j|| of every slot of the chunk (0 past n), as k_stats
    // writes it
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float ss = sqs[tt];
      ss += xor32(ss);
      if (hf == 0) p.inv_norm[head * (long)p.wstride + tok0 + 32 * tt + l32] = inv_norm_of(ss);
    }
  }
  // the keys and the staged queries as opaque values from here: the pooling
  // unpacks and reads them again instead of keeping copies from the partials
  // alive (in scratch) across the waits
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int j = 0; j < NC; ++j) asm volatile("" : "+v"(kf[tt].c[j]));
  asm volatile("" ::: "memory");

  // ---- merged slices (k_reduce's order), by the head's first work-groups
  for (int part = chunk; part < NP; part += nwg) {
    __syncthreads();  // red is free
    if (part < 2) {
      // rows 16 part .. + 15.  Group gi of the 32 (1024 / 32 rows) takes
      // chunks gi, gi + 32, ... in turn; the groups are then merged in
      // order.  Thread (r, q) runs groups q and q + 16 of row 16 part + r.
      const int r = tid & 15, q = tid >> 4, row = 16 * part + r;
      float m[2], s[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        m[k] = -INFINITY;
        s[k] = 0.f;
      }
      for (int base = 0; base < nwg; base += 128) {
        uint64_t v[2][4][2];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint64_t* at = pr + (long)min(q + 16 * k + base + 32 * u, nwg - 1) * W + 2 * row;
            v[k][u][0] = ld_dev(at);
            v[k][u][1] = ld_dev(at + 1);
          }
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = q + 16 * k + base + 32 * u;
            if (c < nwg) {
              const uint64_t* at = pr + (long)c * W + 2 * row;
              const float cm = __uint_as_float(untag_w(at, v[k][u][0], tag, p.err));
              const float cs = __uint_as_float(untag_w(at + 1, v[k][u][1], tag, p.err));
              softmax_merge(m[k], s[k], cm, cs);
            }
          }
      }
      float2* gp = reinterpret_cast<float2*>(red);  // [group][16 rows]
#pragma unroll
      for (int k = 0; k < 2; ++k) gp[(q + 16 * k) * 16 + r] = make_float2(m[k], s[k]);
      vmem_done();  // chunk 0's histogram clearing is done before its rows are published
      __syncthreads();
      // every chunk's words have been read: each work-group of the head has
      // read the epoch
      if (part == 0 && tid == 0) st_dev(fp.epoch + head, ep + 1);
      if (tid < 16) {
        float mm = -INFINITY, ss = 0.f;
        for (int g = 0; g < 32; ++g) softmax_merge(mm, ss, gp[g * 16 + tid].x, gp[g * 16 + tid].y);
        st_dev(mr + 2 * row, tagged(tag, __float_as_uint(mm)));
        st_dev(mr + 2 * row + 1, tagged(tag, __float_as_uint(ss > 0.f ? 1.0f / ss : 0.f)));
      }
    } else {
      // unit-key sums of dimensions 32 (part - 2) .. + 31: group gi of 8
      // (1024 / D) takes chunks gi, gi + 8, ... in blocks of four (a block
      // reaching past the last chunk adds zeros); the groups are then added
      // in order
      const int dim = 32 * (part - 2) + (tid & 31), gi = tid >> 5;
      float a = 0.f;
      for (int base = 0; base < nwg; base += 128) {
        uint64_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = ld_dev(pr + (long)min(gi + base + 8 * u, nwg - 1) * W + 64 + dim);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int c = gi + base + 8 * u;
          if (gi + base + 32 * (u / 4) < nwg)
            a += c < nwg ? __uint_as_float(untag_w(pr + (long)c * W + 64 + dim, v[u], tag, p.err)) : 0.f;
        }
      }
      red[gi * 32 + (tid & 31)] = a;
      __syncthreads();
      if (tid < 32) {
        float t = 0.f;
        for (int g = 0; g < 8; ++g) t += red[g * 32 + tid];
        st_dev(mr + 64 + 32 * (part - 2) + tid, tagged(tag, __float_as_uint(t)));
      }
    }
  }

  // ---- importance, redundancy, Z of this chunk's tokens (k_pool's arithmetic)
  __shared__ float2 rs[32];
  __shared__ __attribute__((aligned(16))) float ssh[D];
  if (tid < (kGram ? 64 : 64 + D)) {
    const uint32_t v = untag_w(mr + tid, ld_dev(mr + tid), tag, p.err);
    if (tid < 64) reinterpret_cast<float*>(rs)[tid] = (tid >> 1) < p.m ? __uint_as_float(v) : 0.f;
    else ssh[tid - 64] = __uint_as_float(v);
  }
  __syncthreads();
  if constexpr (kGram) {
    // importance (k_pool's arithmetic)
    const float inv_m = 1.0f / (float)p.m;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const float imp = token_attention<E, D>(kf[tt], qs, rs, sc2, l32, hf) * inv_m;
      const int tok = tok0 + 32 * tt + l32;
      if (hf == 0 && tok < n) p.i_out[head * p.cap + tok] = imp;
      __builtin_amdgcn_sched_barrier(0);  // one accumulator tile live at a time
    }
    return;
  }
  float imp[2], rd[2], z[2];
  pool_tokens<E, D>(kf, qs, rs, ssh, sqs, n, p.m, sc2, p.lambda, tid, imp, rd, z);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tok = tok0 + 32 * tt + l32;
    if (hf == 0 && tok < n) {
      const long o = head * p.cap + tok;
      p.i_out[o] = imp[tt];
      if (p.r_out) p.r_out[o] = rd[tt];
      p.z_out[o] = z[tt];
      if (hg) atomicAdd(&lh[hist_bin(score_key(z[tt]))], 1u);
    }
  }
  if (hg) {
    __syncthreads();
    for (int t = tid; t < kHistBins; t += 256)
      if (lh[t]) atomicAdd(&hg[t], lh[t]);
  }
}

// One unit per work-group over a grid of (chunk, head, sequence) units, all
// resident at once (the host checks it; unit v = chunk + nchunk (head + Hkv
// sequence)).  A persistent form that ran a larger call in rounds of
// resident work-groups was slower than the separate kernels on 64 sequences
// of 8192 tokens (511 against 463 us): a work-group cannot load its next
// unit's keys while it waits for its head's merge, so rounds do not overlap.
template <typename E, int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void k_scores_fused(ScoresFusedParams fp) {
  const int v = blockIdx.x, hb = v / fp.s.nchunk;
  scores_fused_unit<E, D, MODE>(fp, v - hb * fp.s.nchunk, hb % fp.s.hkv, hb / fp.s.hkv);
}

// Short Gram-form caches: the score units of the one-launch pass (chunk
// partials, merged through tagged words; importance and the key weights)
// and the pair-block Gram units (which weigh keys from their own fragments)
// in one grid.  The score units come first, their count rounded up to a
// multiple of 8 so that the pair units keep their XCD-major placement:
// dispatched before any pair unit, they are resident together, which their
// exchange needs (the host checks that this many work-groups of the kernel
// fit on the device at once); the pair units depend on K alone.
struct ScoresPairsParams {
  ScoresFusedParams f;
  GramParams g;
  int nscore;  // score work-groups, a multiple of 8
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_scores_pairs(ScoresPairsParams sp) {
  const int bx = blockIdx.x;
  if (bx >= sp.nscore) {
    // the pair units, whose rounds set the launch's length, take issue
    // priority over the score units' waves on a shared CU (decode call
    // 39.4-39.6 -> 38.3 us; the reverse measured no change)
    __builtin_amdgcn_s_setprio(2);
    gram_pairs_unit(sp.g, bx - sp.nscore);
    return;
  }
  const int nch = sp.f.s.nchunk;
  if (bx >= nch * sp.f.s.hkv * sp.f.s.b) return;
  const int hb = bx / nch;
  scores_fused_unit<BF16, 128, kModeGram>(sp.f, bx - hb * nch, hb % sp.f.s.hkv, hb / sp.f.s.hkv);
}

static int g_scores_pairs_capacity[64];

bool scores_pairs_fit(const ScoresFusedParams& f) {
  const long nscore = ((long)f.s.nchunk * f.s.hkv * f.s.b + 7) / 8 * 8;
  return grid_fits(k_scores_pairs, g_scores_pairs_capacity, nscore);
}

hipError_t launch_scores_pairs(const ScoresFusedParams& f, const GramParams& g, hipStream_t s, Trace* tr) {
  const long nscore = ((long)f.s.nchunk * f.s.hkv * f.s.b + 7) / 8 * 8;
  const long total = nscore + gram_pair_units(g);
  if (total >= (1L << 31)) return hipErrorInvalidValue;
  const ScoresPairsParams sp{f, g, (int)nscore};
  return launch_k(k_scores_pairs, dim3((unsigned)total), dim3(256), s, tr, sp);
}

static int g_fused_capacity[3][64];

bool fused_fits(const FusedParams& p) {
  const long total = (long)((p.cap + kChunk - 1) / kChunk) * p.hkv * p.b;
  if (p.gpart) return p.evict && grid_fits(k_rkv_fused<BF16, 128, true, true>, g_fused_capacity[2], total);
  if (p.evict) return grid_fits(k_rkv_fused<BF16, 128, true, false>, g_fused_capacity[1], total);
  return grid_fits(k_rkv_fused<BF16, 128, false, false>, g_fused_capacity[0], total);
}

static int g_scores_capacity[2][64];

int scores_fused_grid(int mode, const ScoresFusedParams& p) {
  const long total = (long)p.s.nchunk * p.s.hkv * p.s.b;
  if (total >= (1L << 31)) return 0;
  const bool ok = mode == kModeGram
                      ? grid_fits(k_scores_fused<BF16, 128, kModeGram>, g_scores_capacity[0], total)
                      : grid_fits(k_scores_fused<BF16, 128, kModeKeysum>, g_scores_capacity[1], total);
  return ok ? (int)total : 0;
}

hipError_t launch_scores_fused(int mode, const ScoresFusedParams& p, int grid, hipStream_t s, Trace* tr) {
  if (mode == kModeGram) return launch_k(k_scores_fused<BF16, 128, kModeGram>, dim3(grid), dim3(256), s, tr, p);
  return launch_k(k_scores_fused<BF16, 128, kModeKeysum>, dim3(grid), dim3(256), s, tr, p);
}

}  // namespace kvsel
