// Internal interface between the C-ABI host code (api.hip) and the kernel
// translation units.  Every launcher enqueues on the given stream and returns
// the hipError_t of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace kvsel {

constexpr int kChunk = 256;        // tokens per work-group in the streaming passes

// A sequence length as the kernels use it: clamped into [0, cap].  A length
// outside that range is reported in bit 0 of the error word (len_bad).
__device__ __forceinline__ int clamp_len(int len, int cap) { return len < 0 ? 0 : (len > cap ? cap : len); }
__device__ __forceinline__ bool len_bad(int len, int cap) { return len < 0 || len > cap; }
constexpr int kFuseReduceChunks = 16;

// Calls of at most kActiveFirstMaxB sequences map work-group L of a
// (chunk, head, sequence) grid to the L-th chunk that holds keys, in
// (sequence, head, chunk) order: on a ragged batch the work-groups with work
// are dispatched first and those past the last such chunk exit at once
// (with every sequence at full length the map is the identity).  Returns
// false past the last chunk with keys.
constexpr int kActiveFirstMaxB = 16;
__device__ __forceinline__ bool active_chunk_at(int L, const int32_t* lengths, int b, int hkv, int cap,
                                                int& bi, int& h, int& chunk) {
  int lens[kActiveFirstMaxB];
#pragma unroll
  for (int i = 0; i < kActiveFirstMaxB; ++i) lens[i] = lengths[min(i, b - 1)];
#pragma unroll
  for (int i = 0; i < kActiveFirstMaxB; ++i) {
    const int n = max(0, min(lens[i], cap));  // a negative length holds no keys
    const int nch = i < b ? (n + kChunk - 1) / kChunk : 0;
    if (L < nch * hkv) {
      bi = i;
      h = L / nch;
      chunk = L - h * nch;
      return true;
    }
    L -= nch * hkv;
  }
  return false;
}
// The same for work-group (blockIdx.x, .y, .z) of a (chunk, head, sequence) grid.
__device__ __forceinline__ bool active_chunk(const int32_t* lengths, int b, int hkv, int cap, int nchunk,
                                             int& bi, int& h, int& chunk) {
  return active_chunk_at(blockIdx.x + nchunk * (blockIdx.y + hkv * blockIdx.z), lengths, b, hkv, cap, bi,
                         h, chunk);
}
constexpr int kMaxRows = 128;      // g*w (R-KV) or g (cut) rows, in 32-row tiles
constexpr int kSelectThreads = 1024;
constexpr int kSelectLdsKeys = 32768;
// First-level histogram of score keys: the top kHistBits bits.
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;
// Per head the histogram is followed by a few words of selection state (the
// arrival counter of the threshold kernel's work-groups), zeroed with it.
constexpr int kHistStride = kHistBins + 64;
constexpr int kHistArrive = kHistBins;
__device__ __forceinline__ uint32_t hist_bin(uint32_t key) { return key >> (32 - kHistBits); }

enum ScoreMode { kModeGram = 0, kModeKeysum = 1, kModeCut = 2 };

// ReFreeKV energy term of one attention probability a (a square of at most
// 1): floor(fl32(a*a) * 2^52) as an integer, so that sums are order-free.
// energy_fixed takes x = fl32(a*a) * 2^20 (exact scaling): with hi = floor(x)
// and f = x - hi (exact: Sterbenz for x >= 1, f = x below) the term is
// hi * 2^32 + floor(f * 2^32) (f * 2^32 exact, below 2^32).  Equal to the
// double-precision product floored, for every float square in [0, 1].
__device__ __forceinline__ uint64_t energy_fixed(float x) {
  const uint32_t hi = (uint32_t)x;
  const float f = x - (float)hi;
  const uint32_t lo = (uint32_t)(f * 4294967296.0f);
  return ((uint64_t)hi << 32) | lo;
}
// acc += energy_fixed(x), acc held as two 32-bit words (add with carry)
__device__ __forceinline__ void energy_add(uint32_t& lo_acc, uint32_t& hi_acc, float x) {
  const uint32_t hi = (uint32_t)x;
  const float f = x - (float)hi;
  const uint32_t lo = (uint32_t)(f * 4294967296.0f);
  uint32_t c;
  lo_acc = __builtin_addc(lo_acc, lo, 0u, &c);
  hi_acc = __builtin_addc(hi_acc, hi, c, &c);
}
__device__ __forceinline__ uint64_t energy_term(float a) {
  return energy_fixed(fminf(__fmul_rn(a, a), 1.0f) * 1048576.0f);
}

struct ScoreParams {
  const char* q;            // [b][Hq][w][d]  (cut: [b][Hq][d], w = 1)
  const char* k;            // [b][Hkv][cap][d]
  const int32_t* lengths;   // [b]
  int b, hq, hkv, g, w, m;  // m = g*w query rows per KV head
  int mp;                   // m rounded up to 32
  int cap, nchunk;          // nchunk = ceil(cap / kChunk)
  float scale2;             // log2(e)/sqrt(d): logits in base-2 units
  float lambda;
  // cut mode over the last krows query rows of each q head (krows > 1: row r
  // of a q head sees keys j <= n - krows + r); this launch scores the group
  // of rows rows0 .. rows0 + m - 1 of the g*krows rows of a KV head
  int rows0, krows;
  // workspace
  float2* cstat;            // [b][Hkv][nchunk][mp]  chunk (max, sum 2^(t - max))
  float2* rstat;            // [b][Hkv][mp]          (max, 1/sum), base 2
  float* spart;             // [b][Hkv][nchunk][d]   keysum: chunk sums of unit keys
  float* ssum;              // [b][Hkv][d]           keysum: sum of unit keys
  float* inv_norm;          // [b][Hkv][wstride]     gram: 1/||k_j||, 0 past n in its chunk
  int wstride;              // per-head stride of inv_norm: cap rounded up to 512
  float* logits;            // nullable [b][Hkv][nchunk][m][kChunk]  cut: logits in base-2 units (-inf masked)
  // cut mode, energies formed in k_pool from recomputed logits (no logits buffer)
  uint64_t* energy;         // [b][Hkv][nchunk*kChunk]  integer energy per position
  uint64_t* ctot;           // [b][Hkv][nchunk]          chunk totals of energy
  int accum;                // add to the energies of earlier row groups
  int32_t* err;             // error word
  // R-KV modes with nchunk <= kFuseReduceChunks: k_pool merges the chunk
  // partials itself (in k_reduce's order) and k_reduce is not launched
  int fuse_reduce;
  // outputs (never null; the host substitutes workspace buffers)
  float* i_out;             // [b][Hkv][cap]
  float* r_out;             // [b][Hkv][cap] (may be null in keysum mode)
  float* z_out;             // [b][Hkv][cap]
  uint32_t* hist;           // nullable [b][Hkv][kHistStride]: first-level key histogram of Z
};

struct GramParams {
  const char* k;
  const int32_t* lengths;
  int b, hkv, cap;
  float lambda;
  const float* inv_norm;    // [b][Hkv][wstride]; only positions < n are read as weights
  int wstride;              // per-head stride of inv_norm (multiple of 512)
  const float* i_in;        // [b][Hkv][cap]
  float* r_out;             // nullable
  float* z_out;
  uint32_t* hist;           // nullable [b][Hkv][kHistStride]
  float* rs;                // [b][Hkv][cap]  a key's own-block row sums minus its self term
  float* part;              // [b][Hkv][nsmax][cap]  column sums by block distance - 1
  int nsmax;                // slots per head: (ceil(cap / 256)) / 2, or ceil(cap / 128) when
                            // cap <= kGramPairCap (enough for any block size)
  int bs;                   // symmetric block size of the launched Gram kernel (256 or 512)
  int pairs;                // k_gram_pairs ran: slot s of a key holds its sums against block s
};

// caches of at most this many positions (bf16, d = 128) use k_gram_pairs
constexpr int kGramPairCap = 4096;

constexpr int kSelChunk = 512;     // positions per compaction work-group

// most work-groups that share one selection chunk's gather
constexpr int kMaxGsplit = 8;
struct SelectParams {
  uint32_t salt;            // per-call salt of the one-launch selection's tags (head_tag)
  const float* z;           // [b][Hkv][cap]
  const int32_t* lengths;
  int b, hkv, cap, budget;
  int32_t* idx;             // [b][Hkv][budget]
  uint32_t* hist;           // [b][Hkv][kHistStride]: first-level key histogram of z
  // split select (cap <= kSelectLdsKeys): threshold per head, offsets per chunk
  uint32_t* thr;            // [b][Hkv][4]: threshold key, copies of it to keep, copies in all
  uint32_t* coff;           // [b][Hkv][nsc]: output slot of the chunk's first kept position
  uint32_t* ceqb;           // [b][Hkv][nsc]: keys equal to the threshold before the chunk
  int nsc;                  // ceil(cap / kSelChunk)
  // threshold kernel, per chunk: keys above the first-level bin, and the
  // bin's keys (candidates) with their positions, at the chunk's own offset
  uint32_t* acnt;           // [b][Hkv][nsc]
  uint32_t* ccnt;           // [b][Hkv][nsc]
  uint32_t* candk;          // [b][Hkv][cap]
  int32_t* candp;           // [b][Hkv][cap]
  // one-launch selection and compaction (k_select_compact): tagged words
  // over the memory of candk/candp ([b][Hkv][cap], candidate keys at the
  // chunk's own offset) and of acnt/ccnt ([b][Hkv][nsc], candidates | keys
  // above the bin << 16); the head's epoch is word 3 of its thr record
  uint64_t* cand64;
  uint64_t* cnt64;
  int one_launch;           // the caller allows it (otherwise always two kernels)
  // fused gather (k == nullptr: indices only)
  const char* k;
  const char* v;
  char* k_out;
  char* v_out;
  int cap_out, row_bytes;
  // work-groups sharing one chunk's gather (1 .. kMaxGsplit): each takes its
  // share of the chunk's kept rows; used when most rows are kept
  int gsplit;
  // per-head budgets (nullable): head h keeps budgets[h] clamped to [0, budget],
  // budget being the row stride of idx and of the compacted cache
  const int32_t* budgets;   // [Hkv]
  int32_t* err;             // nullable error word: bit 0 length > cap, bit 1 budget clamped
  // slot reuse (no compaction): evicted slots instead of kept positions
  const int32_t* pos;       // nullable [b][Hkv][cap]: token position held by each slot
  int32_t* evict;           // [b][Hkv][evict_stride]: evicted slots ascending, then -1
  int evict_stride;
  int32_t* n_evict;         // [b][Hkv]
};

struct SlotWriteParams {
  char* k;                  // [b][Hkv][cap][d]
  char* v;
  int32_t* pos;             // nullable [b][Hkv][cap]
  const char* k_new;        // [b][Hkv][count][d]
  const char* v_new;
  const int32_t* pos_new;   // nullable [b]: position of new token 0
  const int32_t* evict;     // [b][Hkv][evict_stride]
  int evict_stride;
  const int32_t* n_evict;   // [b][Hkv]
  int b, hkv, cap, count;
};

struct GatherParams {
  const char* k;
  const char* v;
  const int32_t* idx;       // [b][Hkv][budget]
  int b, hkv, cap, budget, cap_out;
  char* k_out;
  char* v_out;
};

struct CutParams {
  const float* logits;      // [b][Hkv][nchunk][rows][kChunk] (or null with attn)
  const float* attn;        // [b][Hq][cap]           stage entry (or null)
  const float2* rstat;      // [b][Hkv][mp]
  const int32_t* lengths;
  int b, hq, hkv, g, mp, cap, nchunk, n_sink;
  int rows;                 // attention rows per KV head in this launch (g for one last row)
  int accum;                // add to the energies of earlier row groups
  float T;
  uint64_t* energy;         // [b][Hkv][nchunk*kChunk]
  uint64_t* ctot;           // [b][Hkv][nchunk]
  int32_t* kept;            // [b][Hkv]
  int32_t* err;
};

struct CutCompactParams {
  const char* k;            // [b][Hkv][cap][d]
  const char* v;
  char* k_out;              // [b][Hkv][cap_out][d]
  char* v_out;
  const int32_t* lengths;
  const int32_t* kept;      // [b][Hkv]
  int b, hkv, cap, cap_out, n_sink;
};

// One-launch R-KV step for short caches (fused.hip): key-sum redundancy,
// bf16 keys of 128 dimensions, at most 32 window rows per KV head and at most
// kFusedMaxChunks chunks of kChunk tokens per head, every work-group of the
// grid resident at once (the host checks the grid against the device's
// capacity for this kernel before choosing it).
constexpr int kFusedMaxChunks = 16;
constexpr int kFusedWordsA = 64 + 128;  // per chunk: 32 row (max, sum) pairs, 128 unit-key sums
struct FusedParams {
  const char* q;            // [b][Hq][w][d]
  const char* k;            // [b][Hkv][cap][d]
  const char* v;
  const int32_t* lengths;
  int b, hq, hkv, g, w, m;  // m = g*w <= 32
  int cap, budget, cap_out;
  float scale2, lambda;
  const int32_t* budgets;   // nullable [Hkv]
  float* z_out;             // [b][Hkv][cap]
  int32_t* idx;             // [b][Hkv][budget]
  char* k_out;              // [b][Hkv][cap_out][d]
  char* v_out;
  int32_t* err;
  // slot reuse (non-null evict: evicted slots listed instead of the compaction)
  const int32_t* pos;       // nullable [b][Hkv][cap]: token position of each slot
  int32_t* evict;           // [b][Hkv][evict_stride]
  int evict_stride;
  int32_t* n_evict;         // [b][Hkv]
  // Gram form (non-null gpart): Z from the pooling's importance, the key
  // weights and the pair-block Gram slots instead of phases 1 and 2
  const float* gpart;       // [b][Hkv][nsmax][cap]: slot s = sums against block s
  int nsmax;
  const float* inv_norm;    // [b][Hkv][wstride]
  int wstride;
  const float* i_in;        // [b][Hkv][cap]
  // workspace
  uint64_t* epoch;          // [b][Hkv]: advanced by one every call
  uint64_t* flags;          // [2][b][Hkv][kFusedMaxChunks]: barrier flag words
  uint64_t* pub_a;          // [b][Hkv][kFusedMaxChunks][kFusedWordsA]: tagged chunk partials
  uint64_t* pub_b;          // [b][Hkv][cap]: tagged score keys
  uint32_t salt;            // per-call salt of the tags (head_tag)
};

// One-launch score pass (fused.hip): what k_stats, k_reduce and k_pool
// compute, in one grid of kChunk-token work-groups (bf16 keys of 128
// dimensions, at most 32 window rows per KV head), every work-group of the
// grid resident at once: the key-sum scores, or the importance and key
// weights of the Gram form.  Chunk partials and the merged record are tagged
// words: kFusedWordsA per record in the key-sum form (the layout of the
// short-cache step's records), kGramWordsA (the row statistics alone) in the
// Gram form.  The first work-groups of a head each merge one slice (rows
// 0-15, rows 16-31, then in the key-sum form the unit-key sums 32 dimensions
// at a time: kScoreMergeParts slices).
constexpr int kScoreMergeParts = 2 + 128 / 32;
constexpr int kGramWordsA = 64;  // per chunk: 32 row (max, sum) pairs
struct ScoresFusedParams {
  ScoreParams s;            // shapes, inputs, outputs, histogram, error word
  uint64_t* epoch;          // [b][Hkv]: advanced by one every call
  uint64_t* part;           // [b][Hkv][nchunk][words per record]: tagged chunk partials
  uint64_t* merged;         // [b][Hkv][words per record]: tagged merged record
  uint32_t salt;            // per-call salt of the tags (head_tag)
};

// Optional per-kernel timing: the k-th kernel an entry point launches records
// ev[2k] when it starts and ev[2k+1] when it ends (hipExtLaunchKernelGGL).
struct Trace {
  hipEvent_t* ev;
  int n;
  int k;
};

// Debug builds (-DKVSEL_DEBUG, `python -m decode_eviction_amd.build --debug`):
// every launch is followed by a wait on the stream (skipped while the stream
// is being captured), and a failing kernel is named on stderr with its grid,
// so that a fault is reported at the kernel that caused it instead of at a
// later call.
inline hipError_t debug_check(const void* kern, dim3 grid, dim3 block, hipStream_t s, hipError_t e) {
#ifdef KVSEL_DEBUG
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (e == hipSuccess && hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone)
    e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    hipFunction_t f = nullptr;
    const char* name = hipGetFuncBySymbol(&f, kern) == hipSuccess && f ? hipKernelNameRef(f) : nullptr;
    fprintf(stderr, "kvsel: kernel %s, grid %u x %u x %u, block %u: %s\n", name ? name : "(unknown)",
            grid.x, grid.y, grid.z, block.x, hipGetErrorString(e));
  }
#else
  (void)kern;
  (void)grid;
  (void)block;
  (void)s;
#endif
  return e;
}

template <typename F, typename... Args>
inline hipError_t launch_k(F kern, dim3 grid, dim3 block, hipStream_t s, Trace* tr, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (tr) {
    if (2 * tr->k + 1 < tr->n) {
      e0 = tr->ev[2 * tr->k];
      e1 = tr->ev[2 * tr->k + 1];
    }
    tr->k++;
  }
  hipExtLaunchKernelGGL(kern, grid, block, 0, s, e0, e1, 0, args...);
  return debug_check(reinterpret_cast<const void*>(kern), grid, block, s, hipGetLastError());
}

hipError_t launch_stats(int dt, int d, int mode, const ScoreParams& p, hipStream_t s, Trace* tr);
hipError_t launch_reduce(int d, int mode, const ScoreParams& p, hipStream_t s, Trace* tr);
hipError_t launch_pool(int dt, int d, int mode, const ScoreParams& p, hipStream_t s, Trace* tr);
hipError_t launch_gram(int dt, int d, const GramParams& p, hipStream_t s, Trace* tr);
// The Gram parameters of the kernel launch_gram picks (block size, pair form).
GramParams gram_config(int dt, int d, const GramParams& p);
// Work-groups of the pair-block Gram kernel (one per pair of 128-key blocks).
long gram_pair_units(const GramParams& p);
// k_gram_fin alone (after the pair units ran inside k_pool_pairs).
hipError_t launch_gram_fin(const GramParams& p, hipStream_t s, Trace* tr);
// Short Gram-form caches (bf16, d = 128, at most 32 window rows per KV head,
// cap <= kGramPairCap): the importance pooling (with the key weights) and the
// pair-block Gram units (which weigh keys themselves) in one launch, after
// k_stats.
hipError_t launch_pool_pairs(const ScoreParams& p, const GramParams& g, hipStream_t s, Trace* tr);
hipError_t launch_select(const SelectParams& p, hipStream_t s, Trace* tr);
hipError_t launch_hist(const SelectParams& p, hipStream_t s, Trace* tr);
hipError_t launch_select_err_zero(const SelectParams& p, hipStream_t s, Trace* tr);
hipError_t launch_select_slots(const SelectParams& p, hipStream_t s, Trace* tr);
hipError_t launch_slots_write(int dt, int d, const SlotWriteParams& p, hipStream_t s, Trace* tr);
hipError_t launch_gather(int dt, int d, const GatherParams& p, hipStream_t s, Trace* tr);
hipError_t launch_cut_energy(const CutParams& p, hipStream_t s, Trace* tr);
hipError_t launch_cut_scan(const CutParams& p, hipStream_t s, Trace* tr);
hipError_t launch_cut_full(const CutParams& p, hipStream_t s, Trace* tr);
hipError_t launch_cut_compact(int dt, int d, const CutCompactParams& p, hipStream_t s, Trace* tr);
// the fused short-cache step: false when the grid does not fit on the device
// at once (then nothing is launched)
bool fused_fits(const FusedParams& p);
hipError_t launch_fused(const FusedParams& p, hipStream_t s, Trace* tr);
// the one-launch score pass: its grid (one work-group per (chunk, head,
// sequence)), or 0 when those do not all fit on the device at once (then the
// separate kernels run)
int scores_fused_grid(int mode, const ScoresFusedParams& p);
// Short Gram-form caches: the one-launch score units and the pair-block Gram
// units in one grid (k_scores_pairs), when the score units fit on the device
// together.
bool scores_pairs_fit(const ScoresFusedParams& f);
hipError_t launch_scores_pairs(const ScoresFusedParams& f, const GramParams& g, hipStream_t s, Trace* tr);
hipError_t launch_scores_fused(int mode, const ScoresFusedParams& p, int grid, hipStream_t s, Trace* tr);

// Work-groups of kern resident on the device at once (cached per device;
// -1 when the query fails).
template <typename K>
inline bool grid_fits(K kern, int* cache, long grid) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (cache[dev] == 0) {
    int per_cu = 0, ncu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return false;
    cache[dev] = per_cu * ncu > 0 ? per_cu * ncu : -1;
  }
  return cache[dev] > 0 && grid <= cache[dev];
}

}  // namespace kvsel
