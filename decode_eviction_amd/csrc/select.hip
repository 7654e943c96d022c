// Top-budget choice per KV head and gather-compaction.
//
// R-KV joint eviction (QbitAI R-KV article, section "R-KV三步走", joint
// eviction under a KV budget): keep the min(B, n) highest scores Z; equal
// scores keep the lower position; positions are written ascending.
//
// k_select: one 1024-thread work-group per (sequence, KV head).
//  1. Scores become order-preserving 32-bit keys (LDS copy when n <= 32768).
//  2. Range-adaptive radix select: the key interval [lo, hi] known to hold the
//     B-th largest key is split into <= 2048 power-of-two-wide bins, an LDS
//     histogram finds the bin where the count from the top reaches the
//     number still needed, and the interval shrinks to that bin; at most
//     three rounds reach a single key value kth.  Afterwards count(> kth) < B
//     and need_eq = B - count(> kth) copies of kth are kept, lowest positions
//     first.
//  3. Compaction: each wave owns a contiguous range of positions.  A counting
//     pass (wave ballots + popcounts) gives per-wave totals, one barrier
//     exchanges them, and a writing pass places each kept position at
//     (#greater before it) + min(#equal before it, need_eq), so the output is
//     ascending without a sort.
// k_gather: bit copies of the kept K and V rows, 16 bytes per lane.
#include "common.hpp"
#include "kernels.hpp"
#include "scan.hpp"

namespace kvsel {

constexpr int kSelBins = 2048;
constexpr int kLoadUnroll = 8;

// Budget of KV head h: the scalar budget, or budgets[h] clamped to
// [0, budget] (budget is then the row stride of the outputs).
__device__ __forceinline__ int head_budget(const SelectParams& p, int h) {
  if (!p.budgets) return p.budget;
  const int v = p.budgets[h];
  return v < 0 ? 0 : (v > p.budget ? p.budget : v);
}

// Error bits of one (sequence, head): a length above cap (bit 0), a per-head
// budget outside [0, budget] (bit 1).
__device__ __forceinline__ void flag_select_errors(const SelectParams& p, int h, int bi) {
  if (!p.err) return;
  int f = len_bad(p.lengths[bi], p.cap) ? 1 : 0;
  if (p.budgets) {
    const int v = p.budgets[h];
    f |= (v < 0 || v > p.budget) ? 2 : 0;
  }
  if (f) atomicOr(p.err, f);
}

__global__ __launch_bounds__(kSelectThreads) void k_select(SelectParams p) {
  __shared__ uint32_t keys[kSelectLdsKeys];
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t wsum[2][kSelWaves];
  __shared__ uint32_t bc[4];

  const int h = blockIdx.x, bi = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int B = head_budget(p, h);
  const long head = (long)bi * p.hkv + h;
  int32_t* out = p.idx + head * p.budget;
  const float* z = p.z + head * p.cap;
  if (tid == 0) flag_select_errors(p, h, bi);

  if (n <= B) {
    for (int t = tid; t < p.budget; t += kSelectThreads) out[t] = t < n ? t : -1;
    return;
  }
  for (int t = B + tid; t < p.budget; t += kSelectThreads) out[t] = -1;
  if (B == 0) return;
  const bool inl = n <= kSelectLdsKeys;

  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int j0 = tid; j0 < n; j0 += kSelectThreads * kLoadUnroll) {
    float zv[kLoadUnroll];
#pragma unroll
    for (int u = 0; u < kLoadUnroll; ++u) zv[u] = z[min(j0 + u * kSelectThreads, n - 1)];
#pragma unroll
    for (int u = 0; u < kLoadUnroll; ++u) {
      const int j = j0 + u * kSelectThreads;
      if (j < n) {
        const uint32_t key = score_key(zv[u]);
        if (inl) keys[j] = key;
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) {
    wsum[0][wave] = kmin;
    wsum[1][wave] = kmax;
  }
  __syncthreads();
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    lo = min(lo, wsum[0][w]);
    hi = max(hi, wsum[1][w]);
  }
  __syncthreads();

  auto key_at = [&](int j) -> uint32_t { return inl ? keys[j] : score_key(z[j]); };

  uint32_t need = (uint32_t)B;  // keys still to take from [lo, hi]; all keys above hi are taken
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > 11 ? bits - 11 : 0;
    const int nb = (int)(span >> shift) + 1;
    for (int t = tid; t < nb; t += kSelectThreads) hist[t] = 0u;
    __syncthreads();
    for (int j = tid; j < n; j += kSelectThreads) {
      const uint32_t u = key_at(j);
      if (u >= lo && u <= hi) atomicAdd(&hist[(u - lo) >> shift], 1u);
    }
    __syncthreads();
    const uint32_t c0 = 2 * tid < nb ? hist[2 * tid] : 0u;
    const uint32_t c1 = 2 * tid + 1 < nb ? hist[2 * tid + 1] : 0u;
    const uint2 sc = block_scan_u32(c0 + c1, wsum[0], tid);
    const uint32_t above = sc.y - sc.x - (c0 + c1);  // keys in bins above 2t+1
    if (above < need && above + c1 >= need) {
      bc[0] = 2 * tid + 1;
      bc[1] = above;
    } else if (above + c1 < need && above + c1 + c0 >= need) {
      bc[0] = 2 * tid;
      bc[1] = above + c1;
    }
    __syncthreads();
    const uint32_t bin = bc[0];
    need -= bc[1];
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)bin << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
    __syncthreads();
  }
  const uint32_t kth = lo;
  const uint32_t need_eq = need;

  // compaction: wave w owns positions [w*span, (w+1)*span); pass 1 counts,
  // one exchange of wave totals, pass 2 writes.  No barrier inside the passes.
  const int span = ((n + kSelWaves - 1) / kSelWaves + 63) & ~63;
  const int w0 = wave * span, w1 = min(n, w0 + span);
  uint32_t cgt = 0, ceq = 0;
  for (int r0 = w0; r0 < w1; r0 += 64) {
    const int j = r0 + lane;
    const uint32_t u = j < w1 ? key_at(j) : 0u;
    cgt += (uint32_t)__popcll(__ballot(j < w1 && u > kth));
    ceq += (uint32_t)__popcll(__ballot(j < w1 && u == kth));
  }
  if (lane == 0) {
    wsum[0][wave] = cgt;
    wsum[1][wave] = ceq;
  }
  __syncthreads();
  uint32_t gt_run = 0, eq_run = 0;
  for (int w = 0; w < wave; ++w) {
    gt_run += wsum[0][w];
    eq_run += wsum[1][w];
  }
  for (int r0 = w0; r0 < w1; r0 += 64) {
    const int j = r0 + lane;
    const uint32_t u = j < w1 ? key_at(j) : 0u;
    const bool gt = j < w1 && u > kth;
    const bool eq = j < w1 && u == kth;
    const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
    const uint32_t gt_before = gt_run + lanemask_lt_count(bgt, lane);
    const uint32_t eq_before = eq_run + lanemask_lt_count(beq, lane);
    if (gt || (eq && eq_before < need_eq)) {
      const uint32_t pos = gt_before + min(eq_before, need_eq);
      if (pos < (uint32_t)B) out[pos] = j;
    }
    gt_run += (uint32_t)__popcll(bgt);
    eq_run += (uint32_t)__popcll(beq);
  }
}

// Split select for cap <= 32768.
//
// The kernels that produce Z also count its keys into a first-level
// histogram on the top kHistBits bits (hist).  k_select_thresh runs one
// 256-thread work-group per 512-position chunk and head: every work-group
// reads the head's histogram and finds the bin b1 where the count from the
// top reaches B (the same bin in all of them), counts its chunk's keys above
// b1 and writes the chunk's keys inside b1 (the candidates, with their
// positions) to the chunk's own part of a candidate buffer.  It then adds one
// to the head's arrival counter; the work-group that arrives last refines the
// threshold over the head's candidates (radix rounds of 8 bits on an LDS
// histogram until at most 64 candidates remain, then an exact rank), counts
// per chunk the keys above the threshold and equal to it, and writes each
// chunk's first output slot.  No work-group waits for another.  k_compact
// (one 256-thread work-group per chunk and head) gives every kept position
// its ascending output slot with one block scan of packed (greater, equal)
// counts and copies the kept K and V rows (the gather is fused).
constexpr int kRegThreads = 1024;
constexpr int kRegWaves = kRegThreads / kWave;
constexpr int kKeysPerThread = kSelectLdsKeys / kRegThreads;   // 32
constexpr int kChunksPerRound = kRegThreads / kSelChunk;       // 2

// Per-chunk offsets from per-chunk (greater, equal) counts; run by wave 0,
// lane c = chunk c (at most 64 chunks).
__device__ __forceinline__ void write_chunk_offsets(const SelectParams& p, long head, int n,
                                                    uint32_t gt, uint32_t eq, uint32_t kth,
                                                    uint32_t need_eq, int lane) {
  const int nch = (n + kSelChunk - 1) / kSelChunk;
  if (lane >= nch) gt = eq = 0u;
  const uint32_t x = wave_incl_scan(eq);
  const uint32_t eqb = x - eq;
  const uint32_t rem = need_eq > eqb ? need_eq - eqb : 0u;
  const uint32_t kept = gt + min(eq, rem);
  const uint32_t y2 = wave_incl_scan(kept);
  if (lane < nch) {
    p.coff[head * p.nsc + lane] = y2 - kept;
    p.ceqb[head * p.nsc + lane] = eqb;
  }
  const uint32_t eq_all = __shfl(x, 63, 64);  // keys equal to the threshold in all chunks
  if (lane == 0) {
    p.thr[head * 4 + 0] = kth;
    p.thr[head * 4 + 1] = need_eq;
    p.thr[head * 4 + 2] = eq_all;
  }
}

// Orders this wave's LDS accesses.  Lanes of one wave read counters that other
// lanes of the same wave updated atomically; without a fence the compiler may
// treat those reads as unaffected by other lanes and forward a lane's own
// earlier store (for instance the zero it wrote) instead of loading.
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup"); }

// One refinement round of the adaptive radix select over keys supplied by
// `visit(f)` (which calls f(key) for every candidate key of this thread).
// hist: kSelBins counters (zeroed here); returns the new (lo, hi, need).
template <int NW, typename Visit>
__device__ __forceinline__ void refine_round(uint32_t& lo, uint32_t& hi, uint32_t& need,
                                             uint32_t* hist, uint32_t* wsum, uint32_t* bc,
                                             int tid, Visit visit) {
  const uint32_t span = hi - lo;
  const int bits = 32 - __clz(span);
  const int shift = bits > 11 ? bits - 11 : 0;
  const int nb = (int)(span >> shift) + 1;
  __syncthreads();
  for (int t = tid; t < kSelBins; t += NW * kWave) hist[t] = 0u;
  __syncthreads();
  visit([&](uint32_t key) {
    const uint32_t off = key - lo;
    if (off <= span) atomicAdd(&hist[off >> shift], 1u);
  });
  __syncthreads();
  const uint32_t d0 = 2 * tid < nb ? hist[2 * tid] : 0u;
  const uint32_t d1 = 2 * tid + 1 < nb ? hist[2 * tid + 1] : 0u;
  const uint2 sc = block_scan_u32<NW>(d0 + d1, wsum, tid);
  const uint32_t above = sc.y - sc.x - (d0 + d1);
  if (above < need && above + d1 >= need) {
    bc[0] = 2 * tid + 1;
    bc[1] = above;
  } else if (above + d1 < need && above + d1 + d0 >= need) {
    bc[0] = 2 * tid;
    bc[1] = above + d1;
  }
  __syncthreads();
  const uint32_t bin = bc[0];
  need -= bc[1];
  const uint64_t nlo = (uint64_t)lo + ((uint64_t)bin << shift);
  const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
  lo = (uint32_t)nlo;
  hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
}


constexpr int kCandLds = 4096;   // candidates the finishing work-group stages in LDS

__global__ __launch_bounds__(256) void k_select_thresh(SelectParams p) {
  constexpr int NT = 256, NW = NT / kWave;
  __shared__ uint32_t rh[kHistBins];          // refinement histogram (11 bits per round)
  __shared__ uint32_t ck[kCandLds];
  __shared__ int32_t cpo[kCandLds];
  __shared__ uint32_t wsum[2][NW];
  __shared__ uint32_t cpre[65];                // prefix of the per-chunk candidate counts
  __shared__ uint32_t cgt[64], ceq[64];        // per chunk: keys above / equal to the threshold
  __shared__ uint32_t rk[kWave];
  __shared__ int32_t rp[kWave];
  __shared__ uint32_t bc[4];
  __shared__ int last_s;

  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long head = (long)bi * p.hkv + h;
  uint32_t* hg = p.hist + head * kHistStride;
  const int c0 = chunk * kSelChunk;
  // the histogram (8 bins per thread) and the chunk's scores (positions past
  // cap read 0) are requested before the length arrives
  const uint4 hv0 = reinterpret_cast<const uint4*>(hg)[2 * tid];
  const uint4 hv1 = reinterpret_cast<const uint4*>(hg)[2 * tid + 1];
  uint32_t zr[2];
  {
    const __amdgpu_buffer_rsrc_t rz = buf_rsrc(p.z + head * p.cap, (uint32_t)p.cap * 4u);
    zr[0] = buf_ld32(rz, (uint32_t)(c0 + tid) * 4u, 0);
    zr[1] = buf_ld32(rz, (uint32_t)(c0 + NT + tid) * 4u, 0);
  }
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int B = head_budget(p, h);
  if (chunk == 0 && tid == 0) flag_select_errors(p, h, bi);
  if (n <= B || B == 0 || c0 >= n) return;  // k_compact keeps everything (or nothing)
  const int nch = (n + kSelChunk - 1) / kSelChunk;

  // level 1: the bin where the count from the top reaches B; thread t holds
  // bins 8t .. 8t+7 and the count of keys above them
  const uint32_t hb[8] = {hv0.x, hv0.y, hv0.z, hv0.w, hv1.x, hv1.y, hv1.z, hv1.w};
  uint32_t hs = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) hs += hb[i];
  if (tid == 0) bc[0] = bc[1] = 0u;
  {
    const uint2 sc = block_scan_u32<NW>(hs, wsum[0], tid);  // (exclusive prefix, total)
    uint32_t above = sc.y - sc.x - hs;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above < (uint32_t)B && above + hb[i] >= (uint32_t)B) {
        bc[0] = 8 * tid + i;
        bc[1] = above;
      }
      above += hb[i];
    }
    __syncthreads();
  }
  const uint32_t b1 = bc[0];
  const uint32_t need1 = (uint32_t)B - bc[1];  // keys still to take from bin b1

  // this chunk: keys above b1 (counted) and keys in b1 (written out)
  uint32_t key[2];
  bool in[2];
  uint32_t gt = 0;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int pos = c0 + e * NT + tid;
    key[e] = score_key(__uint_as_float(zr[e]));
    const uint32_t kb = hist_bin(key[e]);
    const bool ok = pos < n;
    gt += (ok && kb > b1) ? 1u : 0u;
    in[e] = ok && kb == b1;
  }
  const uint64_t m0 = __ballot(in[0]), m1 = __ballot(in[1]);
  uint32_t gtw = gt;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) gtw += __shfl_xor(gtw, o, 64);
  if (lane == 0) {
    wsum[0][wave] = (uint32_t)(__popcll(m0) + __popcll(m1));
    wsum[1][wave] = gtw;
  }
  __syncthreads();
  uint32_t wbase = 0, ncand = 0, agt = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wbase += w < wave ? wsum[0][w] : 0u;
    ncand += wsum[0][w];
    agt += wsum[1][w];
  }
  // publish (device-scope stores), wait for them, then arrive; the last of
  // the head's nch work-groups finishes
  const long cbase = head * p.cap + c0;
  if (in[0]) {
    const uint32_t slot = wbase + lanemask_lt_count(m0, lane);
    st_dev(p.candk + cbase + slot, key[0]);
    st_dev(p.candp + cbase + slot, c0 + tid);
  }
  if (in[1]) {
    const uint32_t slot = wbase + (uint32_t)__popcll(m0) + lanemask_lt_count(m1, lane);
    st_dev(p.candk + cbase + slot, key[1]);
    st_dev(p.candp + cbase + slot, c0 + NT + tid);
  }
  if (tid == 0) {
    st_dev(p.ccnt + head * p.nsc + chunk, ncand);
    st_dev(p.acnt + head * p.nsc + chunk, agt);
  }
  vmem_done();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(hg + kHistArrive, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    last_s = old == (uint32_t)(nch - 1);
  }
  __syncthreads();
  if (!last_s) return;

  // ---- the head's last work-group: per-chunk counts and candidates
  if (wave == 0) {
    const uint32_t cc = lane < nch ? ld_dev(p.ccnt + head * p.nsc + lane) : 0u;
    const uint32_t ac = lane < nch ? ld_dev(p.acnt + head * p.nsc + lane) : 0u;
    const uint32_t x = wave_incl_scan(cc);
    cpre[lane + 1] = x;
    if (lane == 0) cpre[0] = 0u;
    cgt[lane] = ac;
    ceq[lane] = 0u;
  }
  __syncthreads();
  const uint32_t nc = cpre[nch];
  const bool staged = nc <= (uint32_t)kCandLds;
  // candidate i: chunk c with cpre[c] <= i < cpre[c+1], entry i - cpre[c]
  auto cand_src = [&](uint32_t i) -> long {
    int lo = 0, hi = nch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cpre[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    return head * p.cap + (long)lo * kSelChunk + (i - cpre[lo]);
  };
  if (staged) {
    // four threads per chunk, eight candidates each in flight, at known
    // addresses (the chunk's candidates sit at its own offset)
    const int c = tid >> 2;
    const uint32_t cnt = c < nch ? cpre[c + 1] - cpre[c] : 0u;
    const long src = head * p.cap + (long)c * kSelChunk;
    for (uint32_t e0 = tid & 3; e0 < cnt; e0 += 32) {
      uint32_t kk[8];
      int32_t pp[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t e = min(e0 + 4 * u, cnt - 1);
        kk[u] = ld_dev(p.candk + src + e);
        pp[u] = ld_dev(p.candp + src + e);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t e = e0 + 4 * u;
        if (e < cnt) {
          ck[cpre[c] + e] = kk[u];
          cpo[cpre[c] + e] = pp[u];
        }
      }
    }
    __syncthreads();
  }
  // visit(f): f(key, pos) for every candidate, from LDS or (a bin too large
  // for LDS) from the candidate buffer, eight loads in flight per thread
  auto visit = [&](auto f) {
    if (staged) {
      for (uint32_t i = tid; i < nc; i += NT) f(ck[i], cpo[i]);
      return;
    }
    for (uint32_t i0 = tid; i0 < nc; i0 += 8 * NT) {
      uint32_t kk[8];
      int32_t pp[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t i = i0 + u * NT;
        const long src = cand_src(i < nc ? i : nc - 1);
        kk[u] = ld_dev(p.candk + src);
        pp[u] = ld_dev(p.candp + src);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * NT < nc) f(kk[u], pp[u]);
    }
  };

  // refinement inside bin b1: rounds of 11 bits (thread t: sub-bins 8t ..
  // 8t + 7) until at most 64 candidates remain in [lo, hi]; the bin's 21 low
  // bits take at most two rounds
  uint32_t lo = b1 << (32 - kHistBits);
  uint32_t hi = lo | ((1u << (32 - kHistBits)) - 1u);
  uint32_t need = need1, inr = nc;
  while (lo < hi && inr > (uint32_t)kWave) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > kHistBits ? bits - kHistBits : 0;
    const int nb = (int)(span >> shift) + 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) rh[8 * tid + i] = 0u;
    __syncthreads();
    visit([&](uint32_t k, int32_t) {
      const uint32_t off = k - lo;
      if (off <= span) atomicAdd(&rh[off >> shift], 1u);
    });
    __syncthreads();
    uint32_t hb[8], hs = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hb[i] = 8 * tid + i < nb ? rh[8 * tid + i] : 0u;
      hs += hb[i];
    }
    const uint2 sc = block_scan_u32<NW>(hs, wsum[0], tid);
    uint32_t above = sc.y - sc.x - hs;  // candidates in sub-bins above this thread's
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above < need && above + hb[i] >= need) {
        bc[0] = 8 * tid + i;
        bc[1] = above;
        bc[2] = hb[i];
      }
      above += hb[i];
    }
    __syncthreads();
    const uint32_t bin = bc[0];
    need -= bc[1];
    inr = bc[2];
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)bin << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
    __syncthreads();
  }
  if (lo < hi) {
    // at most 64 candidates in range: wave 0 ranks them (larger key, or
    // equal key at a lower position, first); rank need-1 is the threshold
    if (tid == 0) bc[3] = 0u;
    __syncthreads();
    visit([&](uint32_t k, int32_t pos) {
      if (k >= lo && k <= hi) {
        const uint32_t slot = atomicAdd(&bc[3], 1u);
        if (slot < (uint32_t)kWave) {
          rk[slot] = k;
          rp[slot] = pos;
        }
      }
    });
    __syncthreads();
    if (wave == 0) {
      const uint32_t nr = min(bc[3], (uint32_t)kWave);
      const uint32_t mk = lane < (int)nr ? rk[lane] : 0u;
      const int32_t mpos = lane < (int)nr ? rp[lane] : 0x7fffffff;
      uint32_t rank = 0;
      for (uint32_t c = 0; c < nr; ++c) {
        const uint32_t kc = (uint32_t)__builtin_amdgcn_readlane((int)mk, (int)c);
        const int32_t pc = __builtin_amdgcn_readlane(mpos, (int)c);
        rank += (kc > mk || (kc == mk && pc < mpos)) ? 1u : 0u;
      }
      const uint64_t who = __ballot(lane < (int)nr && rank == need - 1);
      const uint32_t kth = __shfl(mk, __ffsll((unsigned long long)who) - 1, 64);
      const uint32_t gtk = (uint32_t)__popcll(__ballot(lane < (int)nr && mk > kth));
      if (lane == 0) {
        bc[0] = kth;
        bc[1] = need - gtk;  // copies of the threshold key still to keep
      }
    }
    __syncthreads();
    lo = hi = bc[0];
    need = bc[1];
  }
  const uint32_t kth = lo;
  // per chunk: candidates above the threshold and equal to it
  visit([&](uint32_t k, int32_t pos) {
    const int c = pos / kSelChunk;
    if (k > kth) atomicAdd(&cgt[c], 1u);
    else if (k == kth) atomicAdd(&ceq[c], 1u);
  });
  __syncthreads();
  if (wave == 0) write_chunk_offsets(p, head, n, cgt[lane], ceq[lane], kth, need, lane);
}

// One 1024-thread work-group per head, for calls with many heads (the
// per-chunk kernel above re-reads the histogram and passes candidates
// through memory, which a grid of hundreds of heads pays for in rounds of
// work-groups).  It finds the level-1 bin from the histogram, then refines
// inside the bin: thread t holds the keys of positions t + 1024 i (i < 32) in
// registers; the bin's keys (its size is known from the histogram) and their
// positions are compacted into LDS with ballots and the remaining radix
// rounds touch only them; a bin too large for LDS (many ties) is refined over
// the register keys.  Then the per-chunk counts and offsets as above.
constexpr int kCandMax = 8192;

__global__ __launch_bounds__(kRegThreads) void k_select_thresh_head(SelectParams p) {
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t cand_key[kCandMax];
  __shared__ int32_t cand_pos[kCandMax];
  __shared__ uint32_t cnt[kKeysPerThread][kRegWaves];   // keys above the level-1 bin per (round, wave)
  __shared__ uint32_t ccnt[64][2];                       // candidate (greater, equal) per chunk
  __shared__ uint32_t wsum[2][kRegWaves];
  __shared__ uint32_t bc[3];

  const int h = blockIdx.x, bi = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long head = (long)bi * p.hkv + h;
  const float* z = p.z + head * p.cap;
  // the histogram and the scores are requested before the length arrives:
  // scores through a buffer resource over the cache's capacity (positions
  // past cap read 0, past n are masked below), all in flight before use
  const uint2 c01 = reinterpret_cast<const uint2*>(p.hist + head * kHistStride)[tid];
  uint32_t key[kKeysPerThread];
  {
    const __amdgpu_buffer_rsrc_t rz = buf_rsrc(z, (uint32_t)p.cap * 4u);
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) key[i] = buf_ld32(rz, (uint32_t)tid * 4u, (uint32_t)(i * kRegThreads * 4));
  }
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int B = head_budget(p, h);
  if (tid == 0) flag_select_errors(p, h, bi);
  if (n <= B || B == 0) return;  // k_compact keeps everything (or nothing)

  // level 1: the bin (of kHistBins) where the count from the top reaches B;
  // the thread that finds it also records its count
  const uint32_t c0 = c01.x, c1 = c01.y;
  uint32_t need = (uint32_t)B;
  if (tid < 64) ccnt[tid][0] = ccnt[tid][1] = 0u;
  {
    const uint2 sc = block_scan_u32<kRegWaves>(c0 + c1, wsum[0], tid);
    const uint32_t above = sc.y - sc.x - (c0 + c1);
    if (above < need && above + c1 >= need) {
      bc[0] = 2 * tid + 1;
      bc[1] = above;
      bc[2] = c1;
    } else if (above + c1 < need && above + c1 + c0 >= need) {
      bc[0] = 2 * tid;
      bc[1] = above + c1;
      bc[2] = c0;
    }
    __syncthreads();
  }
  const uint32_t b1 = bc[0];
  const uint32_t bin_count = bc[2];
  uint32_t lo = b1 << (32 - kHistBits);
  uint32_t hi = lo | ((1u << (32 - kHistBits)) - 1u);
  need -= bc[1];

  // positions past n get key 0: below every bin a valid score can fall in;
  // rounds (of kRegThreads positions) from nrr on hold no position
  const int nrr = (n + kRegThreads - 1) / kRegThreads;
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i)
    key[i] = tid + i * kRegThreads < n ? score_key(__uint_as_float(key[i])) : 0u;

  if (bin_count <= (uint32_t)kCandMax) {
    // pass 1: per wave, the bin's keys and the keys above the bin (ballots only)
    uint32_t mine = 0, wcand = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) {
      if (i >= nrr) break;
      const uint32_t kb = hist_bin(key[i]);
      const uint64_t babove = __ballot(kb > b1);
      const uint64_t bin = __ballot(kb == b1);
      mine = lane == i ? (uint32_t)__popcll(babove) : mine;
      wcand += (uint32_t)__popcll(bin);
    }
    if (lane < kKeysPerThread) cnt[lane][wave] = mine;
    if (lane == 0) wsum[1][wave] = wcand;
    __syncthreads();
    uint32_t wbase = 0, nc = 0;
#pragma unroll
    for (int w = 0; w < kRegWaves; ++w) {
      const uint32_t t = wsum[1][w];
      wbase += w < wave ? t : 0u;
      nc += t;
    }
    // pass 2: write the candidates (key, position) in wave order
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) {
      if (i >= nrr) break;
      const bool in = hist_bin(key[i]) == b1;
      const uint64_t bin = __ballot(in);
      if (in) {
        const uint32_t slot = wbase + lanemask_lt_count(bin, lane);
        cand_key[slot] = key[i];
        cand_pos[slot] = tid + i * kRegThreads;
      }
      wbase += (uint32_t)__popcll(bin);
    }
    __syncthreads();
    // refinement inside the bin: block-wide histogram rounds over the
    // candidates (each narrows [lo, hi] by 11 bits) until at most 64 of them
    // remain in range; those are gathered and wave 0 ranks them (larger key,
    // or equal key at a lower position, first): rank need-1 is the threshold.
    uint32_t inr = nc;
    while (lo < hi && inr > (uint32_t)kWave) {
      refine_round<kRegWaves>(lo, hi, need, hist, wsum[0], bc, tid, [&](auto f) {
        for (uint32_t c = tid; c < nc; c += kRegThreads) f(cand_key[c]);
      });
      inr = hist[bc[0]];  // candidates in the new range
    }
    if (lo < hi) {
      __shared__ uint32_t rk[kWave];
      __shared__ int32_t rp[kWave];
      __shared__ uint32_t nr_s;
      __syncthreads();
      if (tid == 0) nr_s = 0u;
      __syncthreads();
      for (uint32_t c = tid; c < nc; c += kRegThreads) {
        const uint32_t k = cand_key[c];
        if (k >= lo && k <= hi) {
          const uint32_t slot = atomicAdd(&nr_s, 1u);
          rk[slot] = k;
          rp[slot] = cand_pos[c];
        }
      }
      __syncthreads();
      if (wave == 0) {
        // lane c holds candidate c; each lane counts the candidates ranked
        // before its own, broadcasting them one at a time from registers
        const uint32_t nr = nr_s;
        const uint32_t mk = lane < (int)nr ? rk[lane] : 0u;
        const int32_t mpos = lane < (int)nr ? rp[lane] : 0x7fffffff;
        uint32_t rank = 0;
        for (uint32_t c = 0; c < nr; ++c) {
          const uint32_t kc = (uint32_t)__builtin_amdgcn_readlane((int)mk, (int)c);
          const int32_t pc = __builtin_amdgcn_readlane(mpos, (int)c);
          rank += (kc > mk || (kc == mk && pc < mpos)) ? 1u : 0u;
        }
        const uint64_t who = __ballot(lane < (int)nr && rank == need - 1);
        const uint32_t kth = __shfl(mk, __ffsll((unsigned long long)who) - 1, 64);
        const uint32_t gtk = (uint32_t)__popcll(__ballot(lane < (int)nr && mk > kth));
        if (lane == 0) {
          bc[0] = kth;
          bc[1] = need - gtk;  // copies of the threshold key still to keep
        }
      }
      __syncthreads();
      lo = hi = bc[0];
      need = bc[1];
    }
    const uint32_t kth = lo;
    for (uint32_t c = tid; c < nc; c += kRegThreads) {
      const uint32_t k = cand_key[c];
      const int ch = cand_pos[c] / kSelChunk;
      if (k > kth) atomicAdd(&ccnt[ch][0], 1u);
      else if (k == kth) atomicAdd(&ccnt[ch][1], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t gt = 0, eq = 0;
      // chunk c = round c / 2, waves of half c % 2
      const int i = lane / kChunksPerRound, w0 = (lane % kChunksPerRound) * (kRegWaves / kChunksPerRound);
      if (i < kKeysPerThread) {
#pragma unroll
        for (int w = 0; w < kRegWaves / kChunksPerRound; ++w) gt += cnt[i][w0 + w];
      }
      gt += ccnt[lane][0];
      eq = ccnt[lane][1];
      write_chunk_offsets(p, head, n, gt, eq, kth, need, lane);
    }
    return;
  }

  // large bin (many ties or a narrow spread): refine over the register keys
  while (lo < hi)
    refine_round<kRegWaves>(lo, hi, need, hist, wsum[0], bc, tid, [&](auto f) {
#pragma unroll
      for (int i = 0; i < kKeysPerThread; ++i) f(key[i]);
    });
  const uint32_t kth = lo;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const uint64_t bgt = __ballot(key[i] > kth);
    const uint64_t beq = __ballot(key[i] == kth);
    const uint32_t v = (uint32_t)__popcll(bgt) | ((uint32_t)__popcll(beq) << 16);
    mine = lane == i ? v : mine;
  }
  if (lane < kKeysPerThread) cnt[lane][wave] = mine;
  __syncthreads();
  if (wave == 0) {
    uint32_t gt = 0, eq = 0;
    const int i = lane / kChunksPerRound, w0 = (lane % kChunksPerRound) * (kRegWaves / kChunksPerRound);
    if (i < kKeysPerThread) {
#pragma unroll
      for (int w = 0; w < kRegWaves / kChunksPerRound; ++w) {
        const uint32_t v = cnt[i][w0 + w];
        gt += v & 0xffffu;
        eq += v >> 16;
      }
    }
    write_chunk_offsets(p, head, n, gt, eq, kth, need, lane);
  }
}

__global__ __launch_bounds__(256) void k_compact(SelectParams p) {
  constexpr int PPT = kSelChunk / 256;  // positions per thread
  __shared__ uint32_t wsum[4];
  __shared__ int32_t rows[kSelChunk];   // kept positions by slot - chunk offset
  // gsplit work-groups per chunk: all find the chunk's kept positions, the
  // first writes them, each gathers its share of the rows
  const int gs = max(p.gsplit, 1);
  const int chunk = blockIdx.x / gs, part = blockIdx.x % gs;
  const int h = blockIdx.y, bi = blockIdx.z, tid = threadIdx.x;
  const long head = (long)bi * p.hkv + h;
  const int c0 = chunk * kSelChunk;
  const int p0 = c0 + tid * PPT;
  // the threshold record, the chunk's offsets and its scores are requested
  // before the length arrives (none depends on it; positions are clamped to
  // the cache, and the record is ignored when everything is kept)
  uint32_t kth = p.thr[head * 4 + 0], need_eq = p.thr[head * 4 + 1];
  uint32_t off = p.coff[head * p.nsc + chunk], eqb = p.ceqb[head * p.nsc + chunk];
  const float* z = p.z + head * p.cap;
  float zv[PPT];
#pragma unroll
  for (int e = 0; e < PPT; ++e) zv[e] = z[min(p0 + e, p.cap - 1)];
  const int len = p.lengths[bi];
  const int B = head_budget(p, h);
  // one wait for all of these loads (the compiler would otherwise request the
  // record only after the length and budget have arrived)
  asm volatile("" ::"s"(kth), "s"(need_eq), "s"(off), "s"(eqb), "s"(len), "s"(B));
  const int n = clamp_len(len, p.cap);
  int32_t* out = p.idx + head * p.budget;
  if (chunk == 0 && part == 0)
    for (int t = min(n, B) + tid; t < p.budget; t += 256) out[t] = -1;
  if (c0 >= n || B == 0) return;
  const bool all = n <= B;
  if (all) {
    kth = 0;
    need_eq = 0;
    off = c0;
    eqb = 0;
  }
  bool gt[PPT], eq[PPT];
  uint32_t cg = 0, ce = 0;
  if (!all) {
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      const bool ok = p0 + e < n;
      const uint32_t kk = score_key(zv[e]);
      gt[e] = ok && kk > kth;
      eq[e] = ok && kk == kth;
      cg += gt[e];
      ce += eq[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      gt[e] = p0 + e < n;
      eq[e] = false;
      cg += gt[e];
    }
  }
  // exclusive scan of packed counts over the 256 threads (each field < 2^16)
  const int lane = tid & 63, wave = tid >> 6;
  const uint32_t v = cg | (ce << 16);
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? wsum[w] : 0u;
    total += wsum[w];
  }
  const uint32_t pre = before + x - v;
  const uint32_t rem = need_eq > eqb ? need_eq - eqb : 0u;
  uint32_t gtb = pre & 0xffffu, eqbf = pre >> 16;
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    int r = -1;
    if (gt[e]) {
      r = (int)(gtb + min(eqbf, rem));
      ++gtb;
    } else if (eq[e]) {
      if (eqbf < rem) r = (int)(gtb + eqbf);
      ++eqbf;
    }
    if (r >= 0 && off + r < (uint32_t)B) {
      if (part == 0) out[off + r] = p0 + e;
      rows[r] = p0 + e;
    }
  }
  if (!p.k) return;
  const int kept = (int)((total & 0xffffu) + min(total >> 16, rem));
  const int nkc = min(kept, B - (int)off);
  // this work-group's share of the chunk's kept rows: [rb, nk)
  const int share = (nkc + gs - 1) / gs;
  const int rb = part * share, nk = min(nkc, rb + share);
  __syncthreads();
  // fused gather: row_bytes/16 lanes per row, all loads of a thread issued first
  const int lpr = p.row_bytes / 16, rpi = 256 / lpr;
  const int lr = tid / lpr, lc = tid % lpr;
  constexpr int U = 4;
  for (int r0 = rb + lr; r0 < nk; r0 += rpi * U) {
    u32x4_t kv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(r0 + u * rpi, nk - 1);
      const long src = (head * p.cap + rows[r]) * (long)p.row_bytes + lc * 16;
      kv[u] = ld16(p.k + src);
      vv[u] = ld16(p.v + src);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * rpi;
      if (r < nk) {
        const long dst = (head * p.cap_out + (long)(off + r)) * p.row_bytes + lc * 16;
        *reinterpret_cast<u32x4_t*>(p.k_out + dst) = kv[u];
        *reinterpret_cast<u32x4_t*>(p.v_out + dst) = vv[u];
      }
    }
  }
}

// The threshold kernel for a call: one work-group per chunk and head while
// the grid is small, one per head (k_select_thresh_head) for many heads.
constexpr int kThreshHeadsMany = 64;

// ------------------------------------------------- one-launch selection
//
// k_select_thresh and k_compact in one launch, for calls whose grid is
// resident at once.  As in k_compact, gsplit work-groups share a chunk whose
// kept rows are many (about 64 rows per gathering work-group): all of them
// select and scan the chunk, each gathers its share.  The finishing work-group of
// k_select_thresh, and the launch of k_compact after it, wait on each
// other; here no work-group waits for a finisher.  Every work-group
// publishes its chunk's candidates (the keys in the first-level bin) and
// counts as tagged words, reads those of every chunk of its head, finds the
// threshold itself (the same rounds as k_select_thresh over the same keys,
// so the same threshold in every work-group) and its chunk's output slot from
// the per-chunk counts, and compacts its chunk.  Ties at the final rank are
// ordered by candidate index instead of position: any strict order gives the
// same threshold key and the same number of its copies to keep (which
// copies are kept is decided by position, in the compaction, as in
// k_compact).  Results equal the two-kernel path's bit for bit.
//
// The tags hash the head's epoch (word 3 of its thr record, advanced by
// chunk 0 once it has the count words of every work-group of the head, by
// which time each of them has read the epoch); a poll that exceeds its limit
// sets bit 2 of the error word.
constexpr int kSelFusedCand = 4096;  // candidates staged in LDS (more: read from memory)

__global__ __launch_bounds__(256) void k_select_compact(SelectParams p) {
  constexpr int NT = 256, NW = NT / kWave, PPT = kSelChunk / NT;
  __shared__ uint32_t rh[kHistBins];          // refinement histogram
  __shared__ uint32_t ck[kSelFusedCand];      // staged candidate keys
  __shared__ uint8_t cch[kSelFusedCand];      // and their chunks
  __shared__ uint32_t wsum[2][NW];
  __shared__ uint32_t cpre[65];               // prefix of the per-chunk candidate counts
  __shared__ uint32_t cgt[64], ceq[64];       // per chunk: keys above / equal to the threshold
  __shared__ uint32_t rk[kWave], ri[kWave];
  __shared__ uint32_t bc[4];
  __shared__ uint32_t mine[2];                // this chunk's first output slot, copies of kth before it
  __shared__ int32_t rows[kSelChunk];         // kept positions by slot - chunk offset

  const int gs = max(p.gsplit, 1);
  const int chunk = blockIdx.x / gs, part = blockIdx.x % gs, h = blockIdx.y, bi = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long head = (long)bi * p.hkv + h;
  const uint32_t* hg = p.hist + head * kHistStride;
  const int c0 = chunk * kSelChunk;
  const int p0 = c0 + tid * PPT;
  // the histogram (8 bins per thread), the chunk's scores and the head's
  // epoch are requested before the length arrives
  const uint4 hv0 = reinterpret_cast<const uint4*>(hg)[2 * tid];
  const uint4 hv1 = reinterpret_cast<const uint4*>(hg)[2 * tid + 1];
  const float* zp = p.z + head * p.cap;
  float zv[PPT];
#pragma unroll
  for (int e = 0; e < PPT; ++e) zv[e] = zp[min(p0 + e, p.cap - 1)];
  const uint32_t ep = ld_dev(p.thr + head * 4 + 3);
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int B = head_budget(p, h);
  const bool lead = chunk == 0 && part == 0;
  if (lead && tid == 0) flag_select_errors(p, h, bi);
  int32_t* out = p.idx + head * p.budget;
  if (lead)
    for (int t = min(n, B) + tid; t < p.budget; t += NT) out[t] = -1;
  if (c0 >= n || B == 0) return;
  const int nch = (n + kSelChunk - 1) / kSelChunk;
  const bool all = n <= B;
  uint32_t key[PPT];
#pragma unroll
  for (int e = 0; e < PPT; ++e) key[e] = score_key(zv[e]);
  uint32_t kth = 0u, need_eq = 0u, off = (uint32_t)c0, eqb = 0u;

  if (!all) {
    const uint32_t tag = head_tag(ep, head, p.salt);
    // level 1: the bin where the count from the top reaches B (as in
    // k_select_thresh)
    const uint32_t hb[8] = {hv0.x, hv0.y, hv0.z, hv0.w, hv1.x, hv1.y, hv1.z, hv1.w};
    uint32_t hs = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) hs += hb[i];
    if (tid == 0) bc[0] = bc[1] = 0u;
    {
      const uint2 sc = block_scan_u32<NW>(hs, wsum[0], tid);
      uint32_t above = sc.y - sc.x - hs;
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        if (above < (uint32_t)B && above + hb[i] >= (uint32_t)B) {
          bc[0] = 8 * tid + i;
          bc[1] = above;
        }
        above += hb[i];
      }
      __syncthreads();
    }
    const uint32_t b1 = bc[0];
    const uint32_t need1 = (uint32_t)B - bc[1];

    // this chunk: keys above b1 (counted) and the keys in b1 (published)
    bool in[PPT];
    uint32_t gt = 0;
#pragma unroll
    for (int e = 0; e < PPT; ++e) {
      const bool ok = p0 + e < n;
      const uint32_t kb = hist_bin(key[e]);
      gt += (ok && kb > b1) ? 1u : 0u;
      in[e] = ok && kb == b1;
    }
    const uint64_t m0 = __ballot(in[0]), m1 = __ballot(in[1]);
    uint32_t gtw = gt;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) gtw += __shfl_xor(gtw, o, 64);
    __syncthreads();  // wsum is free
    if (lane == 0) {
      wsum[0][wave] = (uint32_t)(__popcll(m0) + __popcll(m1));
      wsum[1][wave] = gtw;
    }
    __syncthreads();
    uint32_t wbase = 0, ncand = 0, agt = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      wbase += w < wave ? wsum[0][w] : 0u;
      ncand += wsum[0][w];
      agt += wsum[1][w];
    }
    // the chunk's candidates (its first work-group), and a count word from
    // every work-group (word part of the chunk's gs)
    uint64_t* cw = p.cand64 + head * p.cap + c0;
    if (part == 0) {
      if (in[0]) st_dev(cw + wbase + lanemask_lt_count(m0, lane), tagged(tag, key[0]));
      if (in[1]) st_dev(cw + wbase + (uint32_t)__popcll(m0) + lanemask_lt_count(m1, lane), tagged(tag, key[1]));
    }
    const uint64_t* cnt = p.cnt64 + head * p.nsc * gs;
    if (tid == 0) st_dev(p.cnt64 + (head * p.nsc + chunk) * gs + part, tagged(tag, ncand | (agt << 16)));

    // every chunk's counts (wave 0, lane c = chunk c)
    if (wave == 0) {
      uint32_t cc = 0u, ac = 0u;
      if (lane < nch) {
        const uint64_t* at = cnt + (long)lane * gs;
        const uint32_t v = untag_w(at, ld_dev(at), tag, p.err);
        cc = v & 0xffffu;
        ac = v >> 16;
      }
      const uint32_t x = wave_incl_scan(cc);
      cpre[lane + 1] = x;
      if (lane == 0) cpre[0] = 0u;
      cgt[lane] = ac;
      ceq[lane] = 0u;
      if (lead) {
        // the other work-groups of each chunk have published too
        for (int i = lane; i < nch * gs; i += kWave)
          if (i % gs != 0) untag_w(cnt + i, ld_dev(cnt + i), tag, p.err);
        // every work-group of the head has published, so has read the epoch
        if (lane == 0) st_dev(p.thr + head * 4 + 3, ep + 1u);
      }
    }
    __syncthreads();
    const uint32_t nc = cpre[nch];
    const bool staged = nc <= (uint32_t)kSelFusedCand;
    // candidate i: chunk c with cpre[c] <= i < cpre[c+1], entry i - cpre[c]
    auto chunk_of = [&](uint32_t i) -> int {
      int lo = 0, hi = nch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cpre[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      return lo;
    };
    if (staged) {
      // four threads per chunk, eight candidates each in flight
      const int c = tid >> 2;
      const uint32_t cnt = c < nch ? cpre[c + 1] - cpre[c] : 0u;
      const uint64_t* src = p.cand64 + head * p.cap + (long)c * kSelChunk;
      for (uint32_t e0 = tid & 3; e0 < cnt; e0 += 32) {
        uint64_t w8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) w8[u] = ld_dev(src + min(e0 + 4u * u, cnt - 1));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t e = e0 + 4u * u;
          if (e < cnt) {
            ck[cpre[c] + e] = untag_w(src + e, w8[u], tag, p.err);
            cch[cpre[c] + e] = (uint8_t)c;
          }
        }
      }
      __syncthreads();
    }
    // visit(f): f(key, chunk, index) for every candidate, from LDS or (a bin
    // too large for LDS: many ties) from memory, eight loads in flight
    auto visit = [&](auto f) {
      if (staged) {
        for (uint32_t i = tid; i < nc; i += NT) f(ck[i], (int)cch[i], i);
        return;
      }
      for (uint32_t i0 = tid; i0 < nc; i0 += 8 * NT) {
        uint64_t w8[8];
        int c8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t i = min(i0 + u * NT, nc - 1);
          c8[u] = chunk_of(i);
          w8[u] = ld_dev(p.cand64 + head * p.cap + (long)c8[u] * kSelChunk + (i - cpre[c8[u]]));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t i = i0 + u * NT;
          if (i < nc) {
            const uint64_t* at = p.cand64 + head * p.cap + (long)c8[u] * kSelChunk + (i - cpre[c8[u]]);
            f(untag_w(at, w8[u], tag, p.err), c8[u], i);
          }
        }
      }
    };

    // refinement inside bin b1 (as in k_select_thresh)
    uint32_t lo = b1 << (32 - kHistBits);
    uint32_t hi = lo | ((1u << (32 - kHistBits)) - 1u);
    uint32_t need = need1, inr = nc;
    while (lo < hi && inr > (uint32_t)kWave) {
      const uint32_t span = hi - lo;
      const int bits = 32 - __clz(span);
      const int shift = bits > kHistBits ? bits - kHistBits : 0;
      const int nb = (int)(span >> shift) + 1;
#pragma unroll
      for (int i = 0; i < 8; ++i) rh[8 * tid + i] = 0u;
      __syncthreads();
      visit([&](uint32_t k, int, uint32_t) {
        const uint32_t o = k - lo;
        if (o <= span) atomicAdd(&rh[o >> shift], 1u);
      });
      __syncthreads();
      uint32_t hb2[8], hs2 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hb2[i] = 8 * tid + i < nb ? rh[8 * tid + i] : 0u;
        hs2 += hb2[i];
      }
      const uint2 sc = block_scan_u32<NW>(hs2, wsum[0], tid);
      uint32_t above = sc.y - sc.x - hs2;
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        if (above < need && above + hb2[i] >= need) {
          bc[0] = 8 * tid + i;
          bc[1] = above;
          bc[2] = hb2[i];
        }
        above += hb2[i];
      }
      __syncthreads();
      const uint32_t bin = bc[0];
      need -= bc[1];
      inr = bc[2];
      const uint64_t nlo = (uint64_t)lo + ((uint64_t)bin << shift);
      const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
      lo = (uint32_t)nlo;
      hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
      __syncthreads();
    }
    if (lo < hi) {
      // at most 64 candidates in range: wave 0 ranks them (larger key, or
      // equal key at a lower candidate index, first); rank need-1 is the
      // threshold
      if (tid == 0) bc[3] = 0u;
      __syncthreads();
      visit([&](uint32_t k, int, uint32_t i) {
        if (k >= lo && k <= hi) {
          const uint32_t slot = atomicAdd(&bc[3], 1u);
          if (slot < (uint32_t)kWave) {
            rk[slot] = k;
            ri[slot] = i;
          }
        }
      });
      __syncthreads();
      if (wave == 0) {
        const uint32_t nr = min(bc[3], (uint32_t)kWave);
        const uint32_t mk = lane < (int)nr ? rk[lane] : 0u;
        const uint32_t mi = lane < (int)nr ? ri[lane] : 0xffffffffu;
        uint32_t rank = 0;
        for (uint32_t c = 0; c < nr; ++c) {
          const uint32_t kc = (uint32_t)__builtin_amdgcn_readlane((int)mk, (int)c);
          const uint32_t ic = (uint32_t)__builtin_amdgcn_readlane((int)mi, (int)c);
          rank += (kc > mk || (kc == mk && ic < mi)) ? 1u : 0u;
        }
        const uint64_t who = __ballot(lane < (int)nr && rank == need - 1);
        const uint32_t kk = __shfl(mk, __ffsll((unsigned long long)who) - 1, 64);
        const uint32_t gtk = (uint32_t)__popcll(__ballot(lane < (int)nr && mk > kk));
        if (lane == 0) {
          bc[0] = kk;
          bc[1] = need - gtk;
        }
      }
      __syncthreads();
      lo = hi = bc[0];
      need = bc[1];
    }
    kth = lo;
    need_eq = need;
    // per chunk: candidates above the threshold and equal to it
    visit([&](uint32_t k, int c, uint32_t) {
      if (k > kth) atomicAdd(&cgt[c], 1u);
      else if (k == kth) atomicAdd(&ceq[c], 1u);
    });
    __syncthreads();
    if (wave == 0) {
      // chunk offsets as write_chunk_offsets forms them; this chunk's only
      const uint32_t g2 = lane < nch ? cgt[lane] : 0u, e2 = lane < nch ? ceq[lane] : 0u;
      const uint32_t x = wave_incl_scan(e2);
      const uint32_t eqbl = x - e2;
      const uint32_t rem = need_eq > eqbl ? need_eq - eqbl : 0u;
      const uint32_t kept = g2 + min(e2, rem);
      const uint32_t y2 = wave_incl_scan(kept);
      if (lane == chunk) {
        mine[0] = y2 - kept;
        mine[1] = eqbl;
      }
      // the head's threshold record, as k_select_thresh leaves it
      const uint32_t eq_all = __shfl(x, 63, 64);
      if (lead && lane == 0) {
        st_dev(p.thr + head * 4 + 0, kth);
        st_dev(p.thr + head * 4 + 1, need_eq);
        st_dev(p.thr + head * 4 + 2, eq_all);
      }
    }
    __syncthreads();
    off = mine[0];
    eqb = mine[1];
  }

  // ---- compaction of this chunk (k_compact with one work-group per chunk)
  bool gtf[PPT], eqf[PPT];
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    const bool ok = p0 + e < n;
    gtf[e] = all ? ok : (ok && key[e] > kth);
    eqf[e] = !all && ok && key[e] == kth;
    cg += gtf[e];
    ce += eqf[e];
  }
  const uint32_t v = cg | (ce << 16);
  const uint32_t x = wave_incl_scan(v);
  __syncthreads();  // wsum is free
  if (lane == 63) wsum[0][wave] = x;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += w < wave ? wsum[0][w] : 0u;
    total += wsum[0][w];
  }
  const uint32_t pre = before + x - v;
  const uint32_t rem = need_eq > eqb ? need_eq - eqb : 0u;
  uint32_t gtb = pre & 0xffffu, eqbf = pre >> 16;
#pragma unroll
  for (int e = 0; e < PPT; ++e) {
    int r = -1;
    if (gtf[e]) {
      r = (int)(gtb + min(eqbf, rem));
      ++gtb;
    } else if (eqf[e]) {
      if (eqbf < rem) r = (int)(gtb + eqbf);
      ++eqbf;
    }
    if (r >= 0 && off + r < (uint32_t)B) {
      if (part == 0) out[off + r] = p0 + e;
      rows[r] = p0 + e;
    }
  }
  if (!p.k) return;
  const int kept = (int)((total & 0xffffu) + min(total >> 16, rem));
  const int nkc = min(kept, B - (int)off);
  // this work-group's share of the chunk's kept rows: [rb, nk)
  const int share = (nkc + gs - 1) / gs;
  const int rb = part * share, nk = min(nkc, rb + share);
  __syncthreads();
  const int lpr = p.row_bytes / 16, rpi = NT / lpr;
  const int lr = tid / lpr, lc = tid % lpr;
  constexpr int U = 4;
  for (int r0 = rb + lr; r0 < nk; r0 += rpi * U) {
    u32x4_t kv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(r0 + u * rpi, nk - 1);
      const long src = (head * p.cap + rows[r]) * (long)p.row_bytes + lc * 16;
      kv[u] = ld16(p.k + src);
      vv[u] = ld16(p.v + src);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * rpi;
      if (r < nk) {
        const long dst = (head * p.cap_out + (long)(off + r)) * p.row_bytes + lc * 16;
        *reinterpret_cast<u32x4_t*>(p.k_out + dst) = kv[u];
        *reinterpret_cast<u32x4_t*>(p.v_out + dst) = vv[u];
      }
    }
  }
}

static int g_selcompact_capacity[64];

// The one-launch selection runs when the caller allows it, the heads are few
// (many heads take k_select_thresh_head) and the whole grid is resident at
// once.
static bool select_compact_ok(const SelectParams& p) {
  if (!p.one_launch || !p.cand64 || !p.cnt64 || p.gsplit > kMaxGsplit || p.nsc > 64) return false;
  if ((long)p.b * p.hkv >= kThreshHeadsMany) return false;
  return grid_fits(k_select_compact, g_selcompact_capacity, (long)p.nsc * max(p.gsplit, 1) * p.hkv * p.b);
}

// ------------------------------------------------------------- slot reuse
//
// Gather-free eviction (the ThinKV page's argument against compaction: a
// gather rewrites almost the whole cache every time it runs): the cache stays
// in place and the evicted slots are listed for new tokens to overwrite.  A
// slot's token position comes from the caller's position map, so the tie rule
// (equal score: the earlier token is kept) follows positions, not slots.
//
// Tied slots of one head split by token position, for k_evict_slots: an
// adaptive radix select over ~pos (larger for earlier tokens) among the tied
// slots gives the position threshold kth2 and the copies need2 of it to keep
// (by slot order).  Returns, per lane, the tied slots above kth2 (g2m) and at
// kth2 (e2m) as masks over the 32 rounds, and the first rank (r2) of this
// lane's wave among the kth2 copies.  Kept out of line: ties that split are
// rare, and inlined, its registers would spill in the common path.
struct TieSplit {
  uint32_t g2m, e2m, r2, need2;
};

__device__ __noinline__ TieSplit split_ties_by_position(const int32_t* ps, int w0, int lane,
                                                        int wave, int tid, uint32_t eqm,
                                                        uint32_t need_eq, uint32_t* hist,
                                                        uint32_t* wsum, uint32_t* bc,
                                                        uint32_t* wtot) {
  constexpr int S = kKeysPerThread;
  auto kpos = [&](int i) -> uint32_t {
    const int s = w0 + kWave * i + lane;
    return ~(uint32_t)(ps ? ps[s] : s);
  };
  uint32_t lo = 0u, hi = 0xffffffffu, need = need_eq;
  while (lo < hi)
    refine_round<kRegWaves>(lo, hi, need, hist, wsum, bc, tid, [&](auto f) {
      for (int i = 0; i < S; ++i)
        if ((eqm >> i) & 1u) f(kpos(i));
    });
  TieSplit t{0u, 0u, 0u, need};
  uint32_t wc = 0u;
  for (int i = 0; i < S; ++i) {
    bool e2 = false;
    if ((eqm >> i) & 1u) {
      const uint32_t k2 = kpos(i);
      t.g2m |= (k2 > lo ? 1u : 0u) << i;
      e2 = k2 == lo;
    }
    t.e2m |= (e2 ? 1u : 0u) << i;
    wc += (uint32_t)__popcll(__ballot(e2));
  }
  if (lane == 0) wtot[wave] = wc;
  __syncthreads();
  for (int w = 0; w < wave; ++w) t.r2 += wtot[w];
  return t;
}

// k_evict_slots runs after k_select_thresh, which leaves the threshold key
// kth, the number need_eq of slots with key kth to keep and the number of
// such slots.  When only part of the tied slots is kept, the ones with the
// lowest positions are taken: an adaptive radix select over ~pos among the
// tied slots (equal positions, which a well-formed map does not have, fall
// back to slot order).  One 1024-thread work-group per head; wave w owns
// slots 2048w .. 2048w+2047, read 64 at a time (lane l: slot 2048w + 64i + l),
// so loads are coalesced and the evicted list comes out in slot order from
// ballots within the wave and one exchange of wave totals.
__global__ __launch_bounds__(kRegThreads) void k_evict_slots(SelectParams p) {
  constexpr int S = kKeysPerThread;          // rounds of 64 slots per wave
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t wsum[kRegWaves];
  __shared__ uint32_t wtot[2][kRegWaves];
  __shared__ uint32_t bc[2];
  const int h = blockIdx.x, bi = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long head = (long)bi * p.hkv + h;
  const float* z = p.z + head * p.cap;
  const int w0 = wave * S * kWave;
  // the threshold record and the scores are requested before the length
  // arrives: scores through a buffer resource over the cache's capacity
  // (slots past cap read 0, past n are masked below), all in flight before use
  const uint32_t kth = p.thr[head * 4 + 0];
  const uint32_t need_eq = p.thr[head * 4 + 1];
  const uint32_t count_eq = p.thr[head * 4 + 2];
  uint32_t zv[S];
  {
    const __amdgpu_buffer_rsrc_t rz = buf_rsrc(z, (uint32_t)p.cap * 4u);
#pragma unroll
    for (int i = 0; i < S; ++i) zv[i] = buf_ld32(rz, (uint32_t)(w0 + lane) * 4u, (uint32_t)(kWave * 4 * i));
  }
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int B = head_budget(p, h);
  int32_t* out = p.evict + head * p.evict_stride;
  const int ne = n > B ? n - B : 0;
  if (tid == 0) p.n_evict[head] = ne;
  for (int t = ne + tid; t < p.evict_stride; t += kRegThreads) out[t] = -1;
  if (ne == 0) return;
  if (B == 0) {  // everything goes
    for (int t = tid; t < n; t += kRegThreads) out[t] = t;
    return;
  }
  const bool split = need_eq > 0u && need_eq < count_eq;
  const bool keep_eq = need_eq >= count_eq;  // when not split: all tied slots kept, or none
  const int32_t* ps = p.pos ? p.pos + head * p.cap : nullptr;
  // key flags: only bit masks outlive the loop
  uint32_t gtm = 0u, eqm = 0u;
  {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const bool ok = w0 + kWave * i + lane < n;
      const uint32_t key = score_key(__uint_as_float(zv[i]));
      gtm |= (ok && key > kth ? 1u : 0u) << i;
      eqm |= (ok && key == kth ? 1u : 0u) << i;
    }
  }
  // tied slots split by position (rare): kept are the tied slots with ~pos
  // above kth2 and the first need2 (in slot order) with ~pos == kth2
  TieSplit ts{0u, 0u, 0u, 0u};
  if (split) ts = split_ties_by_position(ps, w0, lane, wave, tid, eqm, need_eq, hist, wsum, bc, wtot[0]);
  const uint32_t g2m = ts.g2m, e2m = ts.e2m, need2 = ts.need2;
  uint32_t r2 = ts.r2;
  // evicted flags, counted per wave
  uint32_t evm = 0u, wev = 0u;
  for (int i = 0; i < S; ++i) {
    const bool ok = w0 + kWave * i + lane < n;
    bool kept = (gtm >> i) & 1u;
    if ((eqm >> i) & 1u) kept = split ? ((g2m >> i) & 1u) != 0u : keep_eq;
    if (split) {  // copies of (kth, kth2) in slot order
      const uint64_t b2 = __ballot((e2m >> i) & 1u);
      if ((e2m >> i) & 1u) kept = r2 + lanemask_lt_count(b2, lane) < need2;
      r2 += (uint32_t)__popcll(b2);
    }
    const bool ev = ok && !kept;
    evm |= (ev ? 1u : 0u) << i;
    wev += (uint32_t)__popcll(__ballot(ev));
  }
  if (lane == 0) wtot[1][wave] = wev;
  __syncthreads();
  uint32_t o = 0u;
  for (int w = 0; w < wave; ++w) o += wtot[1][w];
  for (int i = 0; i < S; ++i) {
    const uint64_t be = __ballot((evm >> i) & 1u);
    if ((evm >> i) & 1u) {
      const uint32_t at = o + lanemask_lt_count(be, lane);
      if (at < (uint32_t)ne) out[at] = w0 + kWave * i + lane;
    }
    o += (uint32_t)__popcll(be);
  }
}

static hipError_t launch_thresh(const SelectParams& p, hipStream_t s, Trace* tr) {
  if ((long)p.b * p.hkv >= kThreshHeadsMany)
    return launch_k(k_select_thresh_head, dim3(p.hkv, p.b), dim3(kRegThreads), s, tr, p);
  return launch_k(k_select_thresh, dim3(p.nsc, p.hkv, p.b), dim3(256), s, tr, p);
}

hipError_t launch_select_slots(const SelectParams& p, hipStream_t s, Trace* tr) {
  hipError_t e = launch_thresh(p, s, tr);
  if (e != hipSuccess) return e;
  return launch_k(k_evict_slots, dim3(p.hkv, p.b), dim3(kRegThreads), s, tr, p);
}

// New tokens into evicted slots: token t < min(count, n_evict) of each head
// replaces slot evict[t] (bit copies of its K and V rows) and, with a
// position map, records position pos_new[b] + t there.  One 16-byte piece
// per thread.
template <int RB>
__global__ __launch_bounds__(256) void k_slots_write(SlotWriteParams p) {
  constexpr int CPR = RB / 16;
  constexpr int RPW = 256 / CPR;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int t = blockIdx.x * RPW + threadIdx.x / CPR, c = threadIdx.x % CPR;
  const long head = (long)bi * p.hkv + h;
  if (t >= p.count || t >= p.n_evict[head]) return;
  const int slot = p.evict[head * p.evict_stride + t];
  if (slot < 0 || slot >= p.cap) return;
  const long src = (head * p.count + t) * (long)RB + c * 16;
  const long dst = (head * p.cap + slot) * (long)RB + c * 16;
  const u32x4_t kv = ld16(p.k_new + src), vv = ld16(p.v_new + src);
  *reinterpret_cast<u32x4_t*>(p.k + dst) = kv;
  *reinterpret_cast<u32x4_t*>(p.v + dst) = vv;
  if (c == 0 && p.pos) p.pos[head * p.cap + slot] = p.pos_new[bi] + t;
}

hipError_t launch_slots_write(int dt, int d, const SlotWriteParams& p, hipStream_t s, Trace* tr) {
  const int rb = d * (dt == 0 ? 2 : 4);
  auto go = [&](auto kern, int rpw) {
    return launch_k(kern, dim3((p.count + rpw - 1) / rpw, p.hkv, p.b), dim3(256), s, tr, p);
  };
  switch (rb) {
    case 128: return go(k_slots_write<128>, 256 / 8);
    case 256: return go(k_slots_write<256>, 256 / 16);
    case 512: return go(k_slots_write<512>, 256 / 32);
  }
  return hipErrorInvalidValue;
}

// Stage entry (scores given by the caller): zero, then fill the first-level
// histogram, one 256-thread work-group per 2048 positions.
__global__ __launch_bounds__(256) void k_hist_zero(SelectParams p) {
  const long head = (long)blockIdx.y * p.hkv + blockIdx.x;
  if (p.err && head == 0 && threadIdx.x == 0) *p.err = 0;
  for (int t = threadIdx.x; t < kHistStride; t += 256) p.hist[head * kHistStride + t] = 0u;
}

__global__ __launch_bounds__(256) void k_hist(SelectParams p) {
  __shared__ uint32_t lh[kHistBins];
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z, tid = threadIdx.x;
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int c0 = chunk * 2048;
  if (c0 >= n) return;
  const long head = (long)bi * p.hkv + h;
  const float* z = p.z + head * p.cap;
  for (int t = tid; t < kHistBins; t += 256) lh[t] = 0u;
  __syncthreads();
  float zv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) zv[e] = z[min(c0 + e * 256 + tid, n - 1)];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c0 + e * 256 + tid < n) atomicAdd(&lh[hist_bin(score_key(zv[e]))], 1u);
  __syncthreads();
  for (int t = tid; t < kHistBins; t += 256)
    if (lh[t]) atomicAdd(&p.hist[head * kHistStride + t], lh[t]);
}

hipError_t launch_hist(const SelectParams& p, hipStream_t s, Trace* tr) {
  hipError_t e = launch_k(k_hist_zero, dim3(p.hkv, p.b), dim3(256), s, tr, p);
  if (e != hipSuccess) return e;
  return launch_k(k_hist, dim3((p.cap + 2047) / 2048, p.hkv, p.b), dim3(256), s, tr, p);
}

// Clears the error word of a select-only call that builds no histogram.
__global__ void k_select_err_zero(SelectParams p) {
  if (threadIdx.x == 0) *p.err = 0;
}

hipError_t launch_select_err_zero(const SelectParams& p, hipStream_t s, Trace* tr) {
  return launch_k(k_select_err_zero, dim3(1), dim3(64), s, tr, p);
}

hipError_t launch_select(const SelectParams& p, hipStream_t s, Trace* tr) {
  if (p.cap <= kSelectLdsKeys) {
    if (select_compact_ok(p))
      return launch_k(k_select_compact, dim3(p.nsc * max(p.gsplit, 1), p.hkv, p.b), dim3(256), s, tr, p);
    hipError_t e = launch_thresh(p, s, tr);
    if (e != hipSuccess) return e;
    return launch_k(k_compact, dim3(p.nsc * std::max(p.gsplit, 1), p.hkv, p.b), dim3(256), s, tr, p);
  }
  return launch_k(k_select, dim3(p.hkv, p.b), dim3(kSelectThreads), s, tr, p);
}

// ------------------------------------------------------------------ gather

template <int RB>
__global__ __launch_bounds__(256) void k_gather(GatherParams p) {
  constexpr int CPR = RB / 16;
  constexpr int RPW = 256 / CPR;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int t = blockIdx.x * RPW + threadIdx.x / CPR, c = threadIdx.x % CPR;
  if (t >= p.budget) return;
  const long head = (long)bi * p.hkv + h;
  const int src = p.idx[head * p.budget + t];
  if (src < 0 || src >= p.cap) return;  // -1 padding; out-of-range indices are ignored
  const long si = (head * p.cap + src) * (long)RB + c * 16;
  const long di = (head * p.cap_out + t) * (long)RB + c * 16;
  const u32x4_t kv = ld16(p.k + si);
  const u32x4_t vv = ld16(p.v + si);
  *reinterpret_cast<u32x4_t*>(p.k_out + di) = kv;
  *reinterpret_cast<u32x4_t*>(p.v_out + di) = vv;
}

template <int RB>
static hipError_t gather_t(const GatherParams& p, hipStream_t s, Trace* tr) {
  constexpr int RPW = 256 / (RB / 16);
  return launch_k(k_gather<RB>, dim3((p.budget + RPW - 1) / RPW, p.hkv, p.b), dim3(256), s, tr, p);
}

hipError_t launch_gather(int dt, int d, const GatherParams& p, hipStream_t s, Trace* tr) {
  const int rb = d * (dt == 0 ? 2 : 4);
  switch (rb) {
    case 128: return gather_t<128>(p, s, tr);
    case 256: return gather_t<256>(p, s, tr);
    case 512: return gather_t<512>(p, s, tr);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvsel
