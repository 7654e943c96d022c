// ReFreeKV threshold cut (review "论文综述：ReFreeKV：迈向无阈值的KV缓存压缩",
// section 二: sinks first then newest to oldest; stop once the energy left out
// falls below T; last attention row only; first two layers kept whole).
//
// The last-row logits and their per-row softmax statistics come from k_stats
// / k_reduce (scores.hip, cut mode).  Here:
//   k_cut_energy  per 256-token chunk: a = 2^(t - max) / sum for each of the
//                 query rows of the group, E[j] = sum_q floor(fl32(a*a) * 2^52)
//                 as a 64-bit integer, and the chunk's exact integer total;
//                 with more rows than one launch scores (the last k rows of
//                 each query head), successive launches add their rows' terms;
//   k_cut_scan    per KV head: tau = ceil(E_total * (1 - T)); if the sinks
//                 alone reach tau the cut is m, otherwise a block-wide
//                 inclusive scan walks the chunk totals from the newest chunk
//                 back to the crossing chunk, then the tokens inside it, and
//                 L = m + (number of newest tokens kept).
// All sums are integer, so the result does not depend on summation order.
#include "common.hpp"
#include "kernels.hpp"

namespace kvsel {

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* wsum, int tid) {
  v = wave_sum_u64(v);
  if ((tid & 63) == 0) wsum[tid >> 6] = v;
  __syncthreads();
  const uint64_t t = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return t;
}

__device__ __forceinline__ uint64_t block_incl_scan_u64(uint64_t v, uint64_t* wsum, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  uint64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint64_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();
  return before + x;
}

__device__ __forceinline__ void write_err(const CutParams& p) {
  int f = 0;
  for (int i = 0; i < p.b; ++i) f |= len_bad(p.lengths[i], p.cap) ? 1 : 0;
  *p.err = f;
}

__global__ __launch_bounds__(256) void k_cut_energy(CutParams p) {
  __shared__ uint64_t wsum[4];
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z, tid = threadIdx.x;
  if (p.attn && chunk == 0 && h == 0 && bi == 0 && tid == 0) write_err(p);
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int c0 = chunk * kChunk;
  if (c0 >= n) return;
  const long head = (long)bi * p.hkv + h;
  const int tok = c0 + tid;
  uint64_t* ep = p.energy + head * (long)p.nchunk * kChunk + tok;
  uint64_t e = p.accum ? *ep : 0u;  // row groups after the first add to the earlier ones
  if (tok < n) {
    if (p.attn) {
      for (int q = 0; q < p.rows; ++q)
        e += energy_term(p.attn[((long)bi * p.hq + (long)h * p.g + q) * p.cap + tok]);
    } else {
      // 8 rows at a time, their loads issued before use; a row that sees no
      // key (sum 0) has no attention mass
      constexpr int U = 8;
      const float* lg = p.logits + (head * p.nchunk + chunk) * p.rows * (long)kChunk + tid;
      const float2* rs = p.rstat + head * p.mp;
      for (int q0 = 0; q0 < p.rows; q0 += U) {
        float t[U];
        float2 st[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = min(q0 + u, p.rows - 1);
          t[u] = lg[q * kChunk];
          st[u] = rs[q];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (q0 + u < p.rows) e += energy_term(st[u].y > 0.f ? exp2_fast(t[u] - st[u].x) * st[u].y : 0.f);
      }
    }
  }
  *ep = e;
  const uint64_t tot = block_sum_u64(e, wsum, tid);
  if (tid == 0) p.ctot[head * p.nchunk + chunk] = tot;
}

__global__ __launch_bounds__(256) void k_cut_scan(CutParams p) {
  __shared__ uint64_t wsum[4];
  __shared__ int found;
  __shared__ uint64_t found_above;
  const int h = blockIdx.x, bi = blockIdx.y, tid = threadIdx.x;
  const long head = (long)bi * p.hkv + h;
  const int n = clamp_len(p.lengths[bi], p.cap);
  if (n == 0) {
    if (tid == 0) p.kept[head] = 0;
    return;
  }
  const uint64_t* E = p.energy + head * (long)p.nchunk * kChunk;
  const uint64_t* ct = p.ctot + head * p.nchunk;
  const int nch = (n + kChunk - 1) / kChunk;
  const int m = min(p.n_sink, n);

  // the chunk holding the first non-sink position; its sink part is summed
  // here so that its non-sink energy is its total minus that part
  const int cm = m / kChunk;
  uint64_t tot = 0, esk = 0, esk_cm = 0;
  for (int c = tid; c < nch; c += 256) tot += ct[c];
  for (int j = tid; j < m; j += 256) {
    const uint64_t e = E[j];
    esk += e;
    esk_cm += j >= cm * kChunk ? e : 0u;
  }
  tot = block_sum_u64(tot, wsum, tid);
  esk = block_sum_u64(esk, wsum, tid);
  esk_cm = block_sum_u64(esk_cm, wsum, tid);
  const double taud = ceil((double)tot * (1.0 - (double)p.T));
  const uint64_t tau = (uint64_t)taud;
  // the sinks alone reach tau (with no sinks this happens only when tau is 0,
  // a total energy of 0: then the first queued token already reaches it)
  if (esk >= tau) {
    if (tid == 0) p.kept[head] = max(m, 1);
    return;
  }

  // chunk level: walk chunks newest first over positions >= m
  if (tid == 0) found = -1;
  __syncthreads();
  uint64_t acc = 0;
  for (int r = 0; r * 256 < nch - cm; ++r) {
    const int c = nch - 1 - (r * 256 + tid);
    uint64_t v = 0;
    if (c >= cm) v = c > cm ? ct[c] : ct[c] - esk_cm;
    const uint64_t incl = acc + block_incl_scan_u64(v, wsum, tid);
    if (c >= cm && esk + incl >= tau && esk + incl - v < tau) {
      found = c;
      found_above = incl - v;
    }
    acc = acc + block_sum_u64(v, wsum, tid);
    __syncthreads();
    if (found >= 0) break;
  }
  const int cstar = found;
  if (cstar < 0) {
    if (tid == 0) p.kept[head] = n;
    return;
  }
  // token level inside the crossing chunk, newest first
  const uint64_t above = found_above;
  const int top = min(n, (cstar + 1) * kChunk) - 1;
  const int low = max(m, cstar * kChunk);
  const int pos = top - tid;
  const uint64_t v = pos >= low ? E[pos] : 0;
  __syncthreads();
  if (tid == 0) found = -1;
  __syncthreads();
  const uint64_t incl = above + block_incl_scan_u64(v, wsum, tid);
  if (pos >= low && esk + incl >= tau && esk + incl - v < tau) found = pos;
  __syncthreads();
  if (tid == 0) p.kept[head] = found >= 0 ? m + (n - found) : n;
}

__global__ void k_cut_full(CutParams p) {
  const int h = blockIdx.x, bi = blockIdx.y;
  if (h == 0 && bi == 0 && threadIdx.x == 0) write_err(p);
  if (threadIdx.x == 0) p.kept[(long)bi * p.hkv + h] = clamp_len(p.lengths[bi], p.cap);
}

// Sink + suffix compaction after the cut (the kept set is the m sinks and
// the newest L - m tokens): row t < L of the compacted cache is position t for
// t < min(m, n), else position n - L + t; bit copies of K and V, one 16-byte
// piece per thread.  Rows from L on are left untouched.
template <int RB>
__global__ __launch_bounds__(256) void k_cut_compact(CutCompactParams p) {
  constexpr int CPR = RB / 16;
  constexpr int RPW = 256 / CPR;
  const int h = blockIdx.y, bi = blockIdx.z;
  const int t = blockIdx.x * RPW + threadIdx.x / CPR, c = threadIdx.x % CPR;
  const long head = (long)bi * p.hkv + h;
  const int n = clamp_len(p.lengths[bi], p.cap);
  const int L = min(p.kept[head], n);
  if (t >= L || t >= p.cap_out) return;
  const int ms = min(p.n_sink, n);
  const int src = t < ms ? t : n - L + t;
  const long from = (head * p.cap + src) * (long)RB + c * 16;
  const long to = (head * p.cap_out + t) * (long)RB + c * 16;
  const u32x4_t kv = ld16(p.k + from), vv = ld16(p.v + from);
  *reinterpret_cast<u32x4_t*>(p.k_out + to) = kv;
  *reinterpret_cast<u32x4_t*>(p.v_out + to) = vv;
}

hipError_t launch_cut_compact(int dt, int d, const CutCompactParams& p, hipStream_t s, Trace* tr) {
  const int rb = d * (dt == 0 ? 2 : 4);
  auto go = [&](auto kern, int rpw) {
    return launch_k(kern, dim3((p.cap + rpw - 1) / rpw, p.hkv, p.b), dim3(256), s, tr, p);
  };
  switch (rb) {
    case 128: return go(k_cut_compact<128>, 256 / 8);
    case 256: return go(k_cut_compact<256>, 256 / 16);
    case 512: return go(k_cut_compact<512>, 256 / 32);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_cut_energy(const CutParams& p, hipStream_t s, Trace* tr) {
  return launch_k(k_cut_energy, dim3(p.nchunk, p.hkv, p.b), dim3(256), s, tr, p);
}

hipError_t launch_cut_scan(const CutParams& p, hipStream_t s, Trace* tr) {
  return launch_k(k_cut_scan, dim3(p.hkv, p.b), dim3(256), s, tr, p);
}

hipError_t launch_cut_full(const CutParams& p, hipStream_t s, Trace* tr) {
  return launch_k(k_cut_full, dim3(p.hkv, p.b), dim3(64), s, tr, p);
}

}  // namespace kvsel
