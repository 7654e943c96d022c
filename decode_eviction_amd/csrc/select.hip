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

namespace kvsel {

constexpr int kSelBins = 2048;
constexpr int kSelWaves = kSelectThreads / kWave;
constexpr int kLoadUnroll = 8;

__device__ __forceinline__ uint32_t lanemask_lt_count(uint64_t m, int lane) {
  return (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

// exclusive prefix sum over the NW*64 threads of the block; returns (prefix, total)
template <int NW = kSelWaves>
__device__ __forceinline__ uint2 block_scan_u32(uint32_t v, uint32_t* wsum, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
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

__global__ __launch_bounds__(kSelectThreads) void k_select(SelectParams p) {
  __shared__ uint32_t keys[kSelectLdsKeys];
  __shared__ uint32_t hist[kSelBins];
  __shared__ uint32_t wsum[2][kSelWaves];
  __shared__ uint32_t bc[4];

  const int h = blockIdx.x, bi = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = min(p.lengths[bi], p.cap);
  const int B = p.budget;
  const long head = (long)bi * p.hkv + h;
  int32_t* out = p.idx + head * B;
  const float* z = p.z + head * p.cap;

  if (n <= B) {
    for (int t = tid; t < B; t += kSelectThreads) out[t] = t < n ? t : -1;
    return;
  }
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

// Register-resident variant for cap <= 32768: 512 threads, thread t holds the
// keys of positions t + 512 i (i < 64).  Each wave counts into its own LDS histogram,
// so atomics only contend inside a wave; compaction counts per (round, wave)
// with ballots, scans the 512 packed counts once, then writes.
constexpr int kRegThreads = 512;
constexpr int kRegWaves = kRegThreads / kWave;
constexpr int kKeysPerThread = kSelectLdsKeys / kRegThreads;

__global__ __launch_bounds__(kRegThreads) void k_select_reg(SelectParams p) {
  __shared__ uint32_t sub[kRegWaves][kSelBins];
  __shared__ uint32_t cnt[kKeysPerThread * kRegWaves];
  __shared__ uint32_t wsum[2][kRegWaves];
  __shared__ uint32_t bc[2];

  const int h = blockIdx.x, bi = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = min(p.lengths[bi], p.cap);
  const int B = p.budget;
  const long head = (long)bi * p.hkv + h;
  int32_t* out = p.idx + head * B;
  const float* z = p.z + head * p.cap;
  if (n <= B) {
    for (int t = tid; t < B; t += kRegThreads) out[t] = t < n ? t : -1;
    return;
  }

  // unconditional loads (index clamped into range) so all of them are in
  // flight before the first use
  float zr[kKeysPerThread];
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) zr[i] = z[min(tid + i * kRegThreads, n - 1)];
  uint32_t key[kKeysPerThread];
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) key[i] = tid + i * kRegThreads < n ? score_key(zr[i]) : 0u;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    if (tid + i * kRegThreads < n) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
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
  for (int w = 0; w < kRegWaves; ++w) {
    lo = min(lo, wsum[0][w]);
    hi = max(hi, wsum[1][w]);
  }
  __syncthreads();

  uint32_t need = (uint32_t)B;
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const int bits = 32 - __clz(span);
    const int shift = bits > 11 ? bits - 11 : 0;
    const int nb = (int)(span >> shift) + 1;
    for (int t = lane; t < nb; t += kWave) sub[wave][t] = 0u;
#pragma unroll
    for (int i = 0; i < kKeysPerThread; ++i) {
      const uint32_t u = key[i];
      if (tid + i * kRegThreads < n && u >= lo && u <= hi) atomicAdd(&sub[wave][(u - lo) >> shift], 1u);
    }
    __syncthreads();
    uint32_t c0 = 0, c1 = 0;
    // thread t owns bins 4t .. 4t+3
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (4 * tid + e < nb) {
#pragma unroll
        for (int w = 0; w < kRegWaves; ++w) c[e] += sub[w][4 * tid + e];
      }
    }
    const uint32_t tsum = c[0] + c[1] + c[2] + c[3];
    const uint2 sc = block_scan_u32<kRegWaves>(tsum, wsum[0], tid);
    uint32_t above = sc.y - sc.x - tsum;  // keys in bins above 4t+3
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      if (above < need && above + c[e] >= need) {
        bc[0] = 4 * tid + e;
        bc[1] = above;
      }
      above += c[e];
    }
    __syncthreads();
    const uint32_t bin = bc[0];
    need -= bc[1];
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)bin << shift);
    const uint64_t nhi = nlo + ((1ull << shift) - 1ull);
    lo = (uint32_t)nlo;
    hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
  }
  const uint32_t kth = lo;
  const uint32_t need_eq = need;

  // counts of (greater, equal) per (round i, wave) packed as gt | eq << 16
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const bool ok = tid + i * kRegThreads < n;
    const uint64_t bgt = __ballot(ok && key[i] > kth);
    const uint64_t beq = __ballot(ok && key[i] == kth);
    if (lane == 0) cnt[i * kRegWaves + wave] = (uint32_t)__popcll(bgt) | ((uint32_t)__popcll(beq) << 16);
  }
  __syncthreads();
  const uint32_t mine = cnt[tid];
  const uint2 sc = block_scan_u32<kRegWaves>(mine, wsum[0], tid);
  cnt[tid] = sc.x;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kKeysPerThread; ++i) {
    const int j = tid + i * kRegThreads;
    const bool ok = j < n;
    const bool gt = ok && key[i] > kth;
    const bool eq = ok && key[i] == kth;
    const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
    const uint32_t pre = cnt[i * kRegWaves + wave];
    const uint32_t gt_before = (pre & 0xffffu) + lanemask_lt_count(bgt, lane);
    const uint32_t eq_before = (pre >> 16) + lanemask_lt_count(beq, lane);
    if (gt || (eq && eq_before < need_eq)) {
      const uint32_t pos = gt_before + min(eq_before, need_eq);
      if (pos < (uint32_t)B) out[pos] = j;
    }
  }
}

hipError_t launch_select(const SelectParams& p, hipStream_t s, Trace* tr) {
  if (p.cap <= kSelectLdsKeys)
    return launch_k(k_select_reg, dim3(p.hkv, p.b), dim3(kRegThreads), s, tr, p);
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
