// libkvsel C ABI: argument checks, workspace carving and launch sequences.
// Nothing here allocates memory or keeps state; every launch goes to the
// caller's stream.  The formulas each entry point computes are stated in
// include/kvsel.h.
#include <math.h>
#include <stdlib.h>

#include <unistd.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "../../include/kvsel.h"
#include "kernels.hpp"

using namespace kvsel;

// Workspace of the allocation-free entry point (kvsel_score_evict_static): a
// file-scope device array, one copy per GPU, held until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory; kernels
// receive the address hipGetSymbolAddress returns for the current device,
// looked up once per device and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[KVSEL_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Device address of the current device's scratch array.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}
}  // namespace

namespace {

constexpr size_t kAlign = 256;

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int rows_padded(int m) { return m <= 32 ? 32 : (m <= 64 ? 64 : 128); }

kvsel_status hip_status(hipError_t e) { return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP; }

// KVSEL_SEPARATE_KERNELS=1 in the environment: the key-sum form always runs
// its separate kernels (the one-launch kernels rely on all of their
// work-groups being resident together, which kernels of other streams
// holding compute units for long can prevent; results are the same bits)
bool separate_kernels() {
  const char* e = getenv("KVSEL_SEPARATE_KERNELS");
  return e && e[0] == '1';
}

// Salts of the one-launch kernels' tags (head_tag): a per-process random
// start (the clock and the process id through the SplitMix64 finaliser),
// then an even stride per launch, so that a stale word in a workspace never
// carries the tag of a later call (see head_tag).
static uint32_t next_salt() {
  static std::atomic<uint32_t> next{[] {
    uint64_t x = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                 ((uint64_t)getpid() << 32);
    x += 0x9e3779b97f4a7c15ull;
    x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
    x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
    return (uint32_t)((x ^ (x >> 31)) >> 32);
  }()};
  return next.fetch_add(0x9e3779b8u, std::memory_order_relaxed);
}

#define KV_TRY(expr)                         \
  do {                                       \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return KVSEL_ERR_HIP; \
  } while (0)

constexpr float kLog2e = 1.44269504088896340736f;

// -------------------------------------------------------------- R-KV layout

struct ScoreWs {
  int32_t* err;
  // one-launch kernels: per-head epochs and tagged chunk partials; the
  // short-cache step of the key-sum form also has barrier tokens and tagged
  // score keys, the score pass a tagged merged record per head
  uint64_t* fepoch;
  uint64_t* fflags;
  uint64_t* fpub_a;
  uint64_t* fpub_b;
  uint64_t* fmerged;
  float2* cstat;
  float2* rstat;
  float* spart;
  float* ssum;
  float* inv_norm;
  float* imp;
  float* z;
  float* grs;    // Gram form: own-block row sums
  float* gpart;  // Gram form: column sums from the other blocks
  int nsmax;
  struct {
    uint32_t* hist;
    uint32_t* thr;
    uint32_t* coff;
    uint32_t* ceqb;
    uint32_t* acnt;
    uint32_t* ccnt;
    uint32_t* candk;
    int32_t* candp;
    int nsc;
  } sel;
  size_t bytes;
};

// per-head stride of the inverse-norm buffer: the Gram kernels read weights
// in blocks of up to 512 keys
int gram_wstride(int cap) { return (cap + 511) / 512 * 512; }

// Layout of one call's workspace.  The key-sum form needs the unit-key sums,
// the Gram form the key weights, own-block row sums and column-sum slots;
// each carves only its own (the size query returns the larger of the two).
ScoreWs score_ws(void* base, int b, int hkv, int d, int m, int cap, kvsel_redundancy mode) {
  const size_t heads = (size_t)b * hkv;
  const int nchunk = (cap + kChunk - 1) / kChunk;
  const int mp = rows_padded(m);
  const bool gram = mode == KVSEL_R_GRAM;
  Carver c{static_cast<char*>(base)};
  ScoreWs w{};
  w.err = c.take<int32_t>(64);
  if (gram) {
    // the one-launch score pass (any length: beside the pair units on short
    // caches) and, on short caches, the one-launch finish
    w.fepoch = c.take<uint64_t>(heads);
    w.fpub_a = c.take<uint64_t>(heads * nchunk * kGramWordsA);
    w.fmerged = c.take<uint64_t>(heads * kGramWordsA);
    if (nchunk <= kFusedMaxChunks) {
      // the short-cache step's Gram finish: barrier flags and score keys
      w.fflags = c.take<uint64_t>(2 * heads * kFusedMaxChunks);
      w.fpub_b = c.take<uint64_t>(heads * cap);
    }
  } else {
    w.fepoch = c.take<uint64_t>(heads);
    if (nchunk <= kFusedMaxChunks) {
      w.fflags = c.take<uint64_t>(2 * heads * kFusedMaxChunks);
      w.fpub_a = c.take<uint64_t>(heads * kFusedMaxChunks * kFusedWordsA);
      w.fpub_b = c.take<uint64_t>(heads * cap);
    } else {
      w.fpub_a = c.take<uint64_t>(heads * nchunk * kFusedWordsA);
      w.fmerged = c.take<uint64_t>(heads * kFusedWordsA);
    }
  }
  w.cstat = c.take<float2>(heads * nchunk * mp);
  w.rstat = c.take<float2>(heads * mp);
  if (!gram) {
    w.spart = c.take<float>(heads * nchunk * d);
    w.ssum = c.take<float>(heads * d);
  }
  w.imp = c.take<float>(heads * cap);
  w.z = c.take<float>(heads * cap);
  w.nsmax = cap <= kGramPairCap ? (cap + 127) / 128 : ((cap + 255) / 256) / 2;
  if (gram) {
    w.inv_norm = c.take<float>(heads * gram_wstride(cap));
    w.grs = c.take<float>(heads * cap);
    w.gpart = c.take<float>(heads * (size_t)w.nsmax * cap);
  }
  w.sel.nsc = (cap + kSelChunk - 1) / kSelChunk;
  w.sel.hist = c.take<uint32_t>(heads * kHistStride);
  w.sel.thr = c.take<uint32_t>(heads * 4);
  w.sel.coff = c.take<uint32_t>(heads * w.sel.nsc);
  w.sel.ceqb = c.take<uint32_t>(heads * w.sel.nsc);
  w.sel.acnt = reinterpret_cast<uint32_t*>(c.take<uint64_t>(heads * w.sel.nsc * kMaxGsplit));
  w.sel.ccnt = w.sel.acnt ? w.sel.acnt + heads * w.sel.nsc : nullptr;
  w.sel.candk = reinterpret_cast<uint32_t*>(c.take<uint64_t>(heads * cap));
  w.sel.candp = w.sel.candk ? reinterpret_cast<int32_t*>(w.sel.candk + heads * cap) : nullptr;
  w.bytes = (c.off + kAlign - 1) / kAlign * kAlign;
  return w;
}

kvsel_status check_score_args(kvsel_dtype dt, kvsel_redundancy mode, const void* q,
                              const void* k, const int32_t* lengths, int b, int hq, int hkv,
                              int d, int w, int cap, float lambda) {
  if (dt != KVSEL_BF16 && dt != KVSEL_F32) return KVSEL_ERR_INVALID_ARG;
  if (mode != KVSEL_R_GRAM && mode != KVSEL_R_KEYSUM) return KVSEL_ERR_INVALID_ARG;
  if (!q || !k || !lengths) return KVSEL_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return KVSEL_ERR_INVALID_ARG;
  if (b < 1 || hq < 1 || hkv < 1 || w < 1 || cap < 1) return KVSEL_ERR_INVALID_ARG;
  if (b > 65535 || hkv > 65535 || cap >= (1 << 24)) return KVSEL_ERR_UNSUPPORTED;
  if (hq % hkv != 0) return KVSEL_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return KVSEL_ERR_UNSUPPORTED;
  if ((long)(hq / hkv) * w > kMaxRows) return KVSEL_ERR_UNSUPPORTED;
  if (!(lambda >= 0.f && lambda <= 1.f)) return KVSEL_ERR_INVALID_ARG;
  return KVSEL_OK;
}

kvsel_status run_scores(kvsel_dtype dt, kvsel_redundancy mode, const void* q, const void* k,
                        const int32_t* lengths, int b, int hq, int hkv, int d, int w, int cap,
                        float lambda, float* i_out, float* r_out, float* z_out,
                        uint32_t* hist, const ScoreWs& ws, hipStream_t stream, Trace* tr,
                        bool gram_fin = true) {
  const int g = hq / hkv;
  ScoreParams p{};
  p.q = static_cast<const char*>(q);
  p.k = static_cast<const char*>(k);
  p.lengths = lengths;
  p.b = b;
  p.hq = hq;
  p.hkv = hkv;
  p.g = g;
  p.w = w;
  p.m = g * w;
  p.mp = rows_padded(p.m);
  p.cap = cap;
  p.nchunk = (cap + kChunk - 1) / kChunk;
  p.scale2 = kLog2e / sqrtf((float)d);
  p.lambda = lambda;
  p.cstat = ws.cstat;
  p.rstat = ws.rstat;
  p.spart = ws.spart;
  p.ssum = ws.ssum;
  p.inv_norm = ws.inv_norm;
  p.wstride = gram_wstride(cap);
  p.logits = nullptr;
  p.err = ws.err;
  p.i_out = i_out ? i_out : ws.imp;
  p.r_out = r_out;
  p.z_out = z_out;
  p.hist = hist;
  const int sm = mode == KVSEL_R_GRAM ? kModeGram : kModeKeysum;
  GramParams gp{};
  if (mode == KVSEL_R_GRAM) {
    gp.k = p.k;
    gp.lengths = lengths;
    gp.b = b;
    gp.hkv = hkv;
    gp.cap = cap;
    gp.lambda = lambda;
    gp.inv_norm = ws.inv_norm;
    gp.wstride = p.wstride;
    gp.i_in = p.i_out;
    gp.r_out = r_out;
    gp.z_out = z_out;
    gp.hist = hist;
    gp.rs = ws.grs;
    gp.part = ws.gpart;
    gp.nsmax = ws.nsmax;
  }
  // short Gram-form caches: the pair-block Gram units (which weigh keys
  // themselves) run beside the importance pass, in one launch with the
  // one-launch score units when those fit on the device together, else
  // beside the pooling after k_stats; the same bits either way
  const bool short_gram = mode == KVSEL_R_GRAM && dt == KVSEL_BF16 && d == 128 && p.mp == 32 &&
                          cap <= kGramPairCap && p.nchunk <= kFuseReduceChunks;
  bool scored = false, paired = false;
  if (short_gram && !separate_kernels()) {
    const ScoresFusedParams fp{p, ws.fepoch, ws.fpub_a, ws.fmerged, next_salt()};
    const GramParams gc = gram_config(dt, d, gp);
    if (scores_pairs_fit(fp)) {
      KV_TRY(launch_scores_pairs(fp, gc, stream, tr));
      scored = paired = true;
    }
  }
  // longer caches (more than kFusedMaxChunks chunks per head): one launch
  // reading K once for the scores (the Gram form's importance and key
  // weights), when its grid fits on the device at once.  On shorter caches
  // the separate kernels measured as fast: k_pool merges the partials itself
  // there, so one launch boundary is all a score pass would save, and its
  // two exchanges between work-groups cost as much.
  if (!scored && dt == KVSEL_BF16 && d == 128 && p.m <= 32 && ws.fmerged &&
      p.nchunk > kFusedMaxChunks && !separate_kernels()) {
    const ScoresFusedParams fp{p, ws.fepoch, ws.fpub_a, ws.fmerged, next_salt()};
    const int grid = scores_fused_grid(sm, fp);
    if (grid > 0) {
      KV_TRY(launch_scores_fused(sm, fp, grid, stream, tr));
      scored = true;
    }
  }
  if (!scored) {
    p.fuse_reduce = p.nchunk <= kFuseReduceChunks;
    KV_TRY(launch_stats(dt, d, sm, p, stream, tr));
    if (!p.fuse_reduce) KV_TRY(launch_reduce(d, sm, p, stream, tr));
    if (!short_gram) KV_TRY(launch_pool(dt, d, sm, p, stream, tr));
  }
  if (mode == KVSEL_R_GRAM) {
    if (short_gram) {
      const GramParams gc = gram_config(dt, d, gp);
      if (!paired) KV_TRY(launch_pool_pairs(p, gc, stream, tr));
      if (gram_fin) KV_TRY(launch_gram_fin(gc, stream, tr));
    } else {
      KV_TRY(launch_gram(dt, d, gp, stream, tr));
    }
  }
  return KVSEL_OK;
}

// ------------------------------------------------------------ select layout

struct SelWs {
  int32_t* err;  // first, so that kvsel_workspace_error reads it
  uint32_t* hist;
  uint32_t* thr;
  uint32_t* coff;
  uint32_t* ceqb;
  uint32_t* acnt;
  uint32_t* ccnt;
  uint32_t* candk;
  int32_t* candp;
  int nsc;
};

SelWs carve_select(Carver& c, int b, int hkv, int cap) {
  const size_t heads = (size_t)b * hkv;
  SelWs w;
  w.err = c.take<int32_t>(64);
  w.nsc = (cap + kSelChunk - 1) / kSelChunk;
  w.hist = c.take<uint32_t>(heads * kHistStride);
  w.thr = c.take<uint32_t>(heads * 4);
  w.coff = c.take<uint32_t>(heads * w.nsc);
  w.ceqb = c.take<uint32_t>(heads * w.nsc);
  // per-chunk counts and candidates: each pair one region, which the
  // one-launch selection uses as 64-bit tagged words instead (a count word
  // per work-group: up to kMaxGsplit per chunk)
  w.acnt = reinterpret_cast<uint32_t*>(c.take<uint64_t>(heads * w.nsc * kMaxGsplit));
  w.ccnt = w.acnt ? w.acnt + heads * w.nsc : nullptr;
  w.candk = reinterpret_cast<uint32_t*>(c.take<uint64_t>(heads * cap));
  w.candp = w.candk ? reinterpret_cast<int32_t*>(w.candk + heads * cap) : nullptr;
  return w;
}

// The single-launch short-cache step (key-sum form, bf16, d = 128, at most 32
// window rows per KV head, at most kFusedMaxChunks chunks per head) applies.
static bool fused_step_applies(kvsel_dtype dt, kvsel_redundancy mode, int hq, int hkv, int d,
                               int w, int cap) {
  return mode == KVSEL_R_KEYSUM && dt == KVSEL_BF16 && d == 128 && (hq / hkv) * w <= 32 &&
         (cap + kChunk - 1) / kChunk <= kFusedMaxChunks;
}

// The Gram form's finish inside the short-cache step applies (bf16, d = 128,
// at most 32 window rows per KV head, the pair-block Gram units).
static bool fused_gram_applies(kvsel_dtype dt, kvsel_redundancy mode, int hq, int hkv, int d,
                               int w, int cap) {
  return mode == KVSEL_R_GRAM && dt == KVSEL_BF16 && d == 128 && (hq / hkv) * w <= 32 &&
         cap <= kGramPairCap && (cap + kChunk - 1) / kChunk <= kFusedMaxChunks;
}

// Its parameters shared by the compacting and the slot-reuse forms.
static FusedParams fused_params(const void* q_window, const void* k, const int32_t* lengths, int b,
                                int hq, int hkv, int d, int w, int cap, float lambda, int budget,
                                const int32_t* budgets, float* z, const ScoreWs& ws) {
  FusedParams fp{};
  fp.q = static_cast<const char*>(q_window);
  fp.k = static_cast<const char*>(k);
  fp.lengths = lengths;
  fp.b = b;
  fp.hq = hq;
  fp.hkv = hkv;
  fp.g = hq / hkv;
  fp.w = w;
  fp.m = fp.g * w;
  fp.cap = cap;
  fp.budget = budget;
  fp.scale2 = kLog2e / sqrtf((float)d);
  fp.lambda = lambda;
  fp.budgets = budgets;
  fp.z_out = z;
  fp.err = ws.err;
  fp.epoch = ws.fepoch;
  fp.flags = ws.fflags;
  fp.pub_a = ws.fpub_a;
  fp.pub_b = ws.fpub_b;
  fp.salt = next_salt();
  return fp;
}

// The Gram finish's inputs: the pooling's importance, the key weights and
// the pair-block Gram slots in the workspace.
static void fused_gram_inputs(FusedParams& fp, const ScoreWs& ws, int cap) {
  fp.gpart = ws.gpart;
  fp.nsmax = ws.nsmax;
  fp.inv_norm = ws.inv_norm;
  fp.wstride = gram_wstride(cap);
  fp.i_in = ws.imp;
}

SelectParams select_params(const SelWs& w, const float* z, const int32_t* lengths, int b, int hkv,
                           int cap, int budget, int32_t* idx) {
  SelectParams sp{};
  sp.z = z;
  sp.lengths = lengths;
  sp.b = b;
  sp.hkv = hkv;
  sp.cap = cap;
  sp.budget = budget;
  sp.idx = idx;
  sp.hist = w.hist;
  sp.thr = w.thr;
  sp.coff = w.coff;
  sp.ceqb = w.ceqb;
  sp.nsc = w.nsc;
  sp.acnt = w.acnt;
  sp.ccnt = w.ccnt;
  sp.candk = w.candk;
  sp.candp = w.candp;
  sp.cand64 = reinterpret_cast<uint64_t*>(w.candk);
  sp.cnt64 = reinterpret_cast<uint64_t*>(w.acnt);
  sp.one_launch = separate_kernels() ? 0 : 1;
  sp.err = w.err;
  sp.salt = next_salt();
  return sp;
}

// ---------------------------------------------------------- ReFreeKV layout

struct CutWs {
  int32_t* err;
  float2* cstat;
  float2* rstat;
  float* logits;
  uint64_t* energy;
  uint64_t* ctot;
  size_t bytes;
};

// Row groups of at most this many rows store their logits for k_cut_energy
// (8 bytes per row and position, written and read back); larger groups form
// the energies in k_pool from logits recomputed from Q and K, which costs one
// more read of K (256 bytes per position for bf16, d = 128) instead.
constexpr int kStoredLogitRows = 32;

// rows: attention rows scored per launch (g for the single last row; up to
// kMaxRows of the g*k last rows)
CutWs cut_ws(void* base, int b, int hkv, int rows, int cap) {
  const size_t heads = (size_t)b * hkv;
  const int nchunk = (cap + kChunk - 1) / kChunk;
  const int mp = rows_padded(rows);
  Carver c{static_cast<char*>(base)};
  CutWs w;
  w.err = c.take<int32_t>(64);
  w.cstat = c.take<float2>(heads * nchunk * mp);
  w.rstat = c.take<float2>(heads * mp);
  w.logits = rows <= kStoredLogitRows ? c.take<float>(heads * rows * (size_t)nchunk * kChunk) : nullptr;
  w.energy = c.take<uint64_t>(heads * (size_t)nchunk * kChunk);
  w.ctot = c.take<uint64_t>(heads * nchunk);
  w.bytes = (c.off + kAlign - 1) / kAlign * kAlign;
  return w;
}

}  // namespace

extern "C" {

const char* kvsel_status_string(kvsel_status s) {
  switch (s) {
    case KVSEL_OK: return "ok";
    case KVSEL_ERR_INVALID_ARG: return "invalid argument";
    case KVSEL_ERR_UNSUPPORTED: return "unsupported shape or type";
    case KVSEL_ERR_WORKSPACE: return "workspace too small";
    case KVSEL_ERR_HIP: return "HIP launch or copy failed";
  }
  return "unknown status";
}

size_t kvsel_score_evict_workspace(int b, int hq, int hkv, int d, int w, int cap, int budget) {
  (void)budget;
  if (b < 1 || hq < 1 || hkv < 1 || w < 1 || cap < 1 || (d != 64 && d != 128)) return 0;
  const int m = (hq / hkv) * w;
  const size_t g = score_ws(nullptr, b, hkv, d, m, cap, KVSEL_R_GRAM).bytes;
  const size_t ks = score_ws(nullptr, b, hkv, d, m, cap, KVSEL_R_KEYSUM).bytes;
  return g > ks ? g : ks;
}

kvsel_status kvsel_scores(kvsel_dtype dt, kvsel_redundancy mode, const void* q_window,
                          const void* k, const int32_t* lengths, int b, int hq, int hkv, int d,
                          int w, int cap, float lambda, float* i_out, float* r_out, float* z_out,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
  kvsel_status st = check_score_args(dt, mode, q_window, k, lengths, b, hq, hkv, d, w, cap, lambda);
  if (st != KVSEL_OK) return st;
  if (!z_out) return KVSEL_ERR_INVALID_ARG;
  const ScoreWs need = score_ws(nullptr, b, hkv, d, (hq / hkv) * w, cap, mode);
  if (!workspace || ws_bytes < need.bytes) return KVSEL_ERR_WORKSPACE;
  const ScoreWs ws = score_ws(workspace, b, hkv, d, (hq / hkv) * w, cap, mode);
  return run_scores(dt, mode, q_window, k, lengths, b, hq, hkv, d, w, cap, lambda, i_out, r_out,
                    z_out, nullptr, ws, stream, nullptr);
}

size_t kvsel_select_workspace(int b, int hkv, int cap) {
  if (b < 1 || hkv < 1 || cap < 1) return 0;
  Carver c{nullptr};
  carve_select(c, b, hkv, cap);
  return (c.off + kAlign - 1) / kAlign * kAlign;
}

static kvsel_status select_impl(const float* z, const int32_t* lengths, const int32_t* budgets,
                                int b, int hkv, int cap, int budget, int32_t* idx_out,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!z || !lengths || !idx_out) return KVSEL_ERR_INVALID_ARG;
  if (b < 1 || hkv < 1 || cap < 1 || budget < 1) return KVSEL_ERR_INVALID_ARG;
  if (b > 65535 || hkv > 65535 || cap >= (1 << 24) || budget > 65536) return KVSEL_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < kvsel_select_workspace(b, hkv, cap)) return KVSEL_ERR_WORKSPACE;
  Carver c{static_cast<char*>(workspace)};
  const SelWs w = carve_select(c, b, hkv, cap);
  SelectParams p = select_params(w, z, lengths, b, hkv, cap, budget, idx_out);
  p.budgets = budgets;
  if (cap <= kSelectLdsKeys) KV_TRY(launch_hist(p, stream, nullptr));  // also clears the error word
  else KV_TRY(launch_select_err_zero(p, stream, nullptr));
  return hip_status(launch_select(p, stream, nullptr));
}

kvsel_status kvsel_select_topb(const float* z, const int32_t* lengths, int b, int hkv, int cap,
                               int budget, int32_t* idx_out, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  return select_impl(z, lengths, nullptr, b, hkv, cap, budget, idx_out, workspace, ws_bytes,
                     stream);
}

kvsel_status kvsel_select_topb_heads(const float* z, const int32_t* lengths,
                                     const int32_t* budgets, int b, int hkv, int cap,
                                     int budget_max, int32_t* idx_out, void* workspace,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!budgets) return KVSEL_ERR_INVALID_ARG;
  return select_impl(z, lengths, budgets, b, hkv, cap, budget_max, idx_out, workspace, ws_bytes,
                     stream);
}

// Slot-reuse arguments: the evicted list must hold n - min(B_h, n) <= cap - B
// entries per head (cap with per-head budgets, which may be 0).
static kvsel_status check_slot_args(const int32_t* evict_out, int evict_stride,
                                    const int32_t* n_evict_out, const int32_t* budgets, int cap,
                                    int budget) {
  if (!evict_out || !n_evict_out) return KVSEL_ERR_INVALID_ARG;
  if (cap > kSelectLdsKeys) return KVSEL_ERR_UNSUPPORTED;
  const int need = budgets ? cap : (cap > budget ? cap - budget : 0);
  if (evict_stride < 1 || evict_stride < need) return KVSEL_ERR_INVALID_ARG;
  return KVSEL_OK;
}

kvsel_status kvsel_select_evict_slots(const float* z, const int32_t* lengths, const int32_t* pos,
                                      const int32_t* budgets, int b, int hkv, int cap, int budget,
                                      int32_t* evict_out, int evict_stride, int32_t* n_evict_out,
                                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!z || !lengths) return KVSEL_ERR_INVALID_ARG;
  if (b < 1 || hkv < 1 || cap < 1 || budget < 1) return KVSEL_ERR_INVALID_ARG;
  if (b > 65535 || hkv > 65535 || budget > 65536) return KVSEL_ERR_UNSUPPORTED;
  kvsel_status st = check_slot_args(evict_out, evict_stride, n_evict_out, budgets, cap, budget);
  if (st != KVSEL_OK) return st;
  if (!workspace || ws_bytes < kvsel_select_workspace(b, hkv, cap)) return KVSEL_ERR_WORKSPACE;
  Carver c{static_cast<char*>(workspace)};
  const SelWs w = carve_select(c, b, hkv, cap);
  SelectParams p = select_params(w, z, lengths, b, hkv, cap, budget, nullptr);
  p.budgets = budgets;
  p.pos = pos;
  p.evict = evict_out;
  p.evict_stride = evict_stride;
  p.n_evict = n_evict_out;
  KV_TRY(launch_hist(p, stream, nullptr));  // also clears the error word
  return hip_status(launch_select_slots(p, stream, nullptr));
}

kvsel_status kvsel_slots_write(kvsel_dtype dt, void* k, void* v, int32_t* pos, const void* k_new,
                               const void* v_new, const int32_t* pos_new, const int32_t* evict,
                               int evict_stride, const int32_t* n_evict, int b, int hkv, int d,
                               int cap, int count, hipStream_t stream) {
  if (dt != KVSEL_BF16 && dt != KVSEL_F32) return KVSEL_ERR_INVALID_ARG;
  if (!k || !v || !k_new || !v_new || !evict || !n_evict) return KVSEL_ERR_INVALID_ARG;
  if (pos && !pos_new) return KVSEL_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_new) || !aligned16(v_new))
    return KVSEL_ERR_INVALID_ARG;
  if (b < 1 || hkv < 1 || cap < 1 || count < 0 || evict_stride < 1) return KVSEL_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return KVSEL_ERR_UNSUPPORTED;
  if (b > 65535 || hkv > 65535 || cap >= (1 << 24)) return KVSEL_ERR_UNSUPPORTED;
  if (count == 0) return KVSEL_OK;
  SlotWriteParams p{static_cast<char*>(k), static_cast<char*>(v), pos,
                    static_cast<const char*>(k_new), static_cast<const char*>(v_new), pos_new,
                    evict, evict_stride, n_evict, b, hkv, cap, count};
  return hip_status(launch_slots_write(dt, d, p, stream, nullptr));
}

kvsel_status kvsel_gather(kvsel_dtype dt, const void* k, const void* v, const int32_t* idx, int b,
                          int hkv, int d, int cap, int budget, void* k_out, void* v_out,
                          int cap_out, hipStream_t stream) {
  if (dt != KVSEL_BF16 && dt != KVSEL_F32) return KVSEL_ERR_INVALID_ARG;
  if (!k || !v || !idx || !k_out || !v_out) return KVSEL_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out))
    return KVSEL_ERR_INVALID_ARG;
  if (b < 1 || hkv < 1 || cap < 1 || budget < 1 || cap_out < budget) return KVSEL_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return KVSEL_ERR_UNSUPPORTED;
  if (b > 65535 || hkv > 65535 || cap >= (1 << 24) || budget > 65536) return KVSEL_ERR_UNSUPPORTED;
  GatherParams p{static_cast<const char*>(k), static_cast<const char*>(v), idx, b, hkv, cap, budget,
                 cap_out, static_cast<char*>(k_out), static_cast<char*>(v_out)};
  return hip_status(launch_gather(dt, d, p, stream, nullptr));
}

static kvsel_status score_evict_impl(kvsel_dtype dt, kvsel_redundancy mode, const void* q_window,
                                     const void* k, const void* v, const int32_t* lengths,
                                     const int32_t* budgets, int b,
                                     int hq, int hkv, int d, int w, int cap, float lambda,
                                     int budget, void* k_out, void* v_out, int cap_out,
                                     int32_t* idx_out, float* scores_out, void* workspace,
                                     size_t ws_bytes, hipStream_t stream, Trace* tr) {
  kvsel_status st = check_score_args(dt, mode, q_window, k, lengths, b, hq, hkv, d, w, cap, lambda);
  if (st != KVSEL_OK) return st;
  if (!v || !k_out || !v_out || !idx_out) return KVSEL_ERR_INVALID_ARG;
  if (!aligned16(v) || !aligned16(k_out) || !aligned16(v_out)) return KVSEL_ERR_INVALID_ARG;
  if (budget < 1 || budget > cap_out) return KVSEL_ERR_INVALID_ARG;
  if (budget > 65536) return KVSEL_ERR_UNSUPPORTED;
  const ScoreWs need = score_ws(nullptr, b, hkv, d, (hq / hkv) * w, cap, mode);
  if (!workspace || ws_bytes < need.bytes) return KVSEL_ERR_WORKSPACE;
  const ScoreWs ws = score_ws(workspace, b, hkv, d, (hq / hkv) * w, cap, mode);
  float* z = scores_out ? scores_out : ws.z;
  // short caches, key-sum form: the whole step in one launch when its grid
  // fits on the device at once
  if (fused_step_applies(dt, mode, hq, hkv, d, w, cap)) {
    FusedParams fp = fused_params(q_window, k, lengths, b, hq, hkv, d, w, cap, lambda, budget,
                                  budgets, z, ws);
    fp.v = static_cast<const char*>(v);
    fp.cap_out = cap_out;
    fp.idx = idx_out;
    fp.k_out = static_cast<char*>(k_out);
    fp.v_out = static_cast<char*>(v_out);
    if (!separate_kernels() && fused_fits(fp)) return hip_status(launch_fused(fp, stream, tr));
  }
  uint32_t* hist = cap <= kSelectLdsKeys ? ws.sel.hist : nullptr;
  st = run_scores(dt, mode, q_window, k, lengths, b, hq, hkv, d, w, cap, lambda, nullptr, nullptr,
                  z, hist, ws, stream, tr);
  if (st != KVSEL_OK) return st;
  SelWs sw;
  sw.hist = ws.sel.hist;
  sw.thr = ws.sel.thr;
  sw.coff = ws.sel.coff;
  sw.ceqb = ws.sel.ceqb;
  sw.acnt = ws.sel.acnt;
  sw.ccnt = ws.sel.ccnt;
  sw.candk = ws.sel.candk;
  sw.candp = ws.sel.candp;
  sw.nsc = ws.sel.nsc;
  sw.err = ws.err;  // set by the first score kernel; the select kernels add to it
  SelectParams sp = select_params(sw, z, lengths, b, hkv, cap, budget, idx_out);
  sp.budgets = budgets;
  if (cap <= kSelectLdsKeys) {  // the compaction kernel also gathers the kept rows
    sp.k = static_cast<const char*>(k);
    sp.v = static_cast<const char*>(v);
    sp.k_out = static_cast<char*>(k_out);
    sp.v_out = static_cast<char*>(v_out);
    sp.cap_out = cap_out;
    sp.row_bytes = d * (dt == KVSEL_BF16 ? 2 : 4);
    // about 64 kept rows per gathering work-group: a chunk of kSelChunk
    // positions keeps about kSelChunk * budget / cap of them
    const long kept_chunk = ((long)kSelChunk * budget + cap - 1) / cap;
    sp.gsplit = (int)std::min((long)kMaxGsplit, std::max(1L, (kept_chunk + 63) / 64));
    KV_TRY(launch_select(sp, stream, tr));
    return KVSEL_OK;
  }
  KV_TRY(launch_select(sp, stream, tr));
  GatherParams gp{static_cast<const char*>(k), static_cast<const char*>(v), idx_out, b, hkv, cap,
                  budget, cap_out, static_cast<char*>(k_out), static_cast<char*>(v_out)};
  KV_TRY(launch_gather(dt, d, gp, stream, tr));
  return KVSEL_OK;
}

kvsel_status kvsel_score_evict(kvsel_dtype dt, kvsel_redundancy mode, const void* q_window,
                               const void* k, const void* v, const int32_t* lengths, int b, int hq,
                               int hkv, int d, int w, int cap, float lambda, int budget,
                               void* k_out, void* v_out, int cap_out, int32_t* idx_out,
                               float* scores_out, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  return score_evict_impl(dt, mode, q_window, k, v, lengths, nullptr, b, hq, hkv, d, w, cap, lambda,
                          budget, k_out, v_out, cap_out, idx_out, scores_out, workspace, ws_bytes,
                          stream, nullptr);
}

kvsel_status kvsel_score_evict_static(kvsel_dtype dt, kvsel_redundancy mode,
                                      const void* q_window, const void* k, const void* v,
                                      const int32_t* lengths, int b, int hq, int hkv, int d, int w,
                                      int cap, float lambda, int budget, void* k_out, void* v_out,
                                      int cap_out, int32_t* idx_out, float* scores_out,
                                      hipStream_t stream) {
  kvsel_status st = check_score_args(dt, mode, q_window, k, lengths, b, hq, hkv, d, w, cap, lambda);
  if (st != KVSEL_OK) return st;
  if (score_ws(nullptr, b, hkv, d, (hq / hkv) * w, cap, mode).bytes > KVSEL_STATIC_SCRATCH_BYTES)
    return KVSEL_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return KVSEL_ERR_HIP;
  return score_evict_impl(dt, mode, q_window, k, v, lengths, nullptr, b, hq, hkv, d, w, cap, lambda,
                          budget, k_out, v_out, cap_out, idx_out, scores_out, ws,
                          KVSEL_STATIC_SCRATCH_BYTES, stream, nullptr);
}

kvsel_status kvsel_score_evict_heads(kvsel_dtype dt, kvsel_redundancy mode, const void* q_window,
                                     const void* k, const void* v, const int32_t* lengths,
                                     const int32_t* budgets, int b, int hq, int hkv, int d, int w,
                                     int cap, float lambda, int budget_max, void* k_out,
                                     void* v_out, int cap_out, int32_t* idx_out,
                                     float* scores_out, void* workspace, size_t ws_bytes,
                                     hipStream_t stream) {
  if (!budgets) return KVSEL_ERR_INVALID_ARG;
  return score_evict_impl(dt, mode, q_window, k, v, lengths, budgets, b, hq, hkv, d, w, cap,
                          lambda, budget_max, k_out, v_out, cap_out, idx_out, scores_out,
                          workspace, ws_bytes, stream, nullptr);
}

kvsel_status kvsel_score_evict_traced(kvsel_dtype dt, kvsel_redundancy mode, const void* q_window,
                                      const void* k, const void* v, const int32_t* lengths, int b,
                                      int hq, int hkv, int d, int w, int cap, float lambda,
                                      int budget, void* k_out, void* v_out, int cap_out,
                                      int32_t* idx_out, float* scores_out, void* workspace,
                                      size_t ws_bytes, hipStream_t stream, hipEvent_t* events,
                                      int n_events) {
  if (!events || n_events < 2) return KVSEL_ERR_INVALID_ARG;
  Trace tr{events, n_events, 0};
  return score_evict_impl(dt, mode, q_window, k, v, lengths, nullptr, b, hq, hkv, d, w, cap, lambda,
                          budget, k_out, v_out, cap_out, idx_out, scores_out, workspace, ws_bytes,
                          stream, &tr);
}

kvsel_status kvsel_score_evict_heads_traced(kvsel_dtype dt, kvsel_redundancy mode,
                                            const void* q_window, const void* k, const void* v,
                                            const int32_t* lengths, const int32_t* budgets, int b,
                                            int hq, int hkv, int d, int w, int cap, float lambda,
                                            int budget_max, void* k_out, void* v_out, int cap_out,
                                            int32_t* idx_out, float* scores_out, void* workspace,
                                            size_t ws_bytes, hipStream_t stream,
                                            hipEvent_t* events, int n_events) {
  if (!budgets || !events || n_events < 2) return KVSEL_ERR_INVALID_ARG;
  Trace tr{events, n_events, 0};
  return score_evict_impl(dt, mode, q_window, k, v, lengths, budgets, b, hq, hkv, d, w, cap,
                          lambda, budget_max, k_out, v_out, cap_out, idx_out, scores_out,
                          workspace, ws_bytes, stream, &tr);
}

static kvsel_status score_evict_slots_impl(kvsel_dtype dt, kvsel_redundancy mode,
                                           const void* q_window, const void* k,
                                           const int32_t* lengths, const int32_t* pos,
                                           const int32_t* budgets, int b, int hq, int hkv, int d,
                                           int w, int cap, float lambda, int budget,
                                           int32_t* evict_out, int evict_stride,
                                           int32_t* n_evict_out, float* scores_out,
                                           void* workspace, size_t ws_bytes, hipStream_t stream,
                                           Trace* tr) {
  kvsel_status st = check_score_args(dt, mode, q_window, k, lengths, b, hq, hkv, d, w, cap, lambda);
  if (st != KVSEL_OK) return st;
  if (budget < 1) return KVSEL_ERR_INVALID_ARG;
  if (budget > 65536) return KVSEL_ERR_UNSUPPORTED;
  st = check_slot_args(evict_out, evict_stride, n_evict_out, budgets, cap, budget);
  if (st != KVSEL_OK) return st;
  const ScoreWs need = score_ws(nullptr, b, hkv, d, (hq / hkv) * w, cap, mode);
  if (!workspace || ws_bytes < need.bytes) return KVSEL_ERR_WORKSPACE;
  const ScoreWs ws = score_ws(workspace, b, hkv, d, (hq / hkv) * w, cap, mode);
  float* z = scores_out ? scores_out : ws.z;
  // short caches, key-sum form: scores, threshold and the evicted list in
  // one launch when its grid fits on the device at once
  if (fused_step_applies(dt, mode, hq, hkv, d, w, cap)) {
    FusedParams fp = fused_params(q_window, k, lengths, b, hq, hkv, d, w, cap, lambda, budget,
                                  budgets, z, ws);
    fp.pos = pos;
    fp.evict = evict_out;
    fp.evict_stride = evict_stride;
    fp.n_evict = n_evict_out;
    if (!separate_kernels() && fused_fits(fp)) return hip_status(launch_fused(fp, stream, tr));
  }
  // short caches, Gram form: the score kernels up to the Gram units, then
  // the finish, threshold and the evicted list in one launch (for the
  // compaction the separate finish and the one-launch selection, whose
  // gather is spread over more work-groups, measured faster)
  if (fused_gram_applies(dt, mode, hq, hkv, d, w, cap) && !separate_kernels()) {
    FusedParams fp = fused_params(q_window, k, lengths, b, hq, hkv, d, w, cap, lambda, budget,
                                  budgets, z, ws);
    fused_gram_inputs(fp, ws, cap);
    fp.pos = pos;
    fp.evict = evict_out;
    fp.evict_stride = evict_stride;
    fp.n_evict = n_evict_out;
    if (fused_fits(fp)) {
      st = run_scores(dt, mode, q_window, k, lengths, b, hq, hkv, d, w, cap, lambda, nullptr,
                      nullptr, z, nullptr, ws, stream, tr, false);
      if (st != KVSEL_OK) return st;
      return hip_status(launch_fused(fp, stream, tr));
    }
  }
  st = run_scores(dt, mode, q_window, k, lengths, b, hq, hkv, d, w, cap, lambda, nullptr, nullptr,
                  z, ws.sel.hist, ws, stream, tr);
  if (st != KVSEL_OK) return st;
  SelWs sw;
  sw.hist = ws.sel.hist;
  sw.thr = ws.sel.thr;
  sw.coff = ws.sel.coff;
  sw.ceqb = ws.sel.ceqb;
  sw.acnt = ws.sel.acnt;
  sw.ccnt = ws.sel.ccnt;
  sw.candk = ws.sel.candk;
  sw.candp = ws.sel.candp;
  sw.nsc = ws.sel.nsc;
  sw.err = ws.err;
  SelectParams sp = select_params(sw, z, lengths, b, hkv, cap, budget, nullptr);
  sp.budgets = budgets;
  sp.pos = pos;
  sp.evict = evict_out;
  sp.evict_stride = evict_stride;
  sp.n_evict = n_evict_out;
  return hip_status(launch_select_slots(sp, stream, tr));
}

kvsel_status kvsel_score_evict_slots(kvsel_dtype dt, kvsel_redundancy mode, const void* q_window,
                                     const void* k, const int32_t* lengths, const int32_t* pos,
                                     const int32_t* budgets, int b, int hq, int hkv, int d, int w,
                                     int cap, float lambda, int budget, int32_t* evict_out,
                                     int evict_stride, int32_t* n_evict_out, float* scores_out,
                                     void* workspace, size_t ws_bytes, hipStream_t stream) {
  return score_evict_slots_impl(dt, mode, q_window, k, lengths, pos, budgets, b, hq, hkv, d, w,
                                cap, lambda, budget, evict_out, evict_stride, n_evict_out,
                                scores_out, workspace, ws_bytes, stream, nullptr);
}

kvsel_status kvsel_score_evict_slots_traced(kvsel_dtype dt, kvsel_redundancy mode,
                                            const void* q_window, const void* k,
                                            const int32_t* lengths, const int32_t* pos,
                                            const int32_t* budgets, int b, int hq, int hkv, int d,
                                            int w, int cap, float lambda, int budget,
                                            int32_t* evict_out, int evict_stride,
                                            int32_t* n_evict_out, float* scores_out,
                                            void* workspace, size_t ws_bytes, hipStream_t stream,
                                            hipEvent_t* events, int n_events) {
  if (!events || n_events < 2) return KVSEL_ERR_INVALID_ARG;
  Trace tr{events, n_events, 0};
  return score_evict_slots_impl(dt, mode, q_window, k, lengths, pos, budgets, b, hq, hkv, d, w,
                                cap, lambda, budget, evict_out, evict_stride, n_evict_out,
                                scores_out, workspace, ws_bytes, stream, &tr);
}

// attention rows scored per launch for the last k_rows rows of each query head
static int cut_group_rows(int g, int k_rows) {
  const long r = (long)g * k_rows;
  return r < kMaxRows ? (int)r : kMaxRows;
}

size_t kvsel_threshold_cut_workspace(int b, int hq, int hkv, int d, int cap) {
  (void)d;
  if (b < 1 || hq < 1 || hkv < 1 || cap < 1 || hq % hkv) return 0;
  return cut_ws(nullptr, b, hkv, hq / hkv, cap).bytes;
}

size_t kvsel_threshold_cut_rows_workspace(int b, int hq, int hkv, int d, int cap, int k_rows) {
  (void)d;
  if (b < 1 || hq < 1 || hkv < 1 || cap < 1 || hq % hkv || k_rows < 1) return 0;
  return cut_ws(nullptr, b, hkv, cut_group_rows(hq / hkv, k_rows), cap).bytes;
}

static kvsel_status check_cut_common(const int32_t* lengths, int b, int hq, int hkv, int cap,
                                     int n_sink, float T, const int32_t* kept) {
  if (!lengths || !kept) return KVSEL_ERR_INVALID_ARG;
  if (b < 1 || hq < 1 || hkv < 1 || cap < 1 || n_sink < 0) return KVSEL_ERR_INVALID_ARG;
  if (hq % hkv != 0) return KVSEL_ERR_INVALID_ARG;
  if (b > 65535 || hkv > 65535 || cap >= (1 << 24)) return KVSEL_ERR_UNSUPPORTED;
  if (hq / hkv > 32) return KVSEL_ERR_UNSUPPORTED;
  if (!(T >= 0.f && T < 1.f)) return KVSEL_ERR_INVALID_ARG;
  return KVSEL_OK;
}

static CutParams cut_params(const CutWs& ws, const int32_t* lengths, int b, int hq, int hkv,
                            int cap, int n_sink, float T, int32_t* kept) {
  CutParams c{};
  c.rstat = ws.rstat;
  c.lengths = lengths;
  c.b = b;
  c.hq = hq;
  c.hkv = hkv;
  c.g = hq / hkv;
  c.mp = rows_padded(c.g);
  c.cap = cap;
  c.nchunk = (cap + kChunk - 1) / kChunk;
  c.n_sink = n_sink;
  c.rows = c.g;
  c.accum = 0;
  c.T = T;
  c.energy = ws.energy;
  c.ctot = ws.ctot;
  c.kept = kept;
  c.err = ws.err;
  return c;
}

// The cut over the last k_rows query rows of each query head (k_rows = 1: the
// single last row), optionally followed by the sink + suffix compaction.
static kvsel_status threshold_cut_impl(kvsel_dtype dt, const void* q_rows, int k_rows,
                                       const void* k, const void* v, const int32_t* lengths,
                                       int b, int hq, int hkv, int d, int cap, int layer,
                                       int n_full_layers, int n_sink, float T,
                                       int32_t* kept_len_out, void* k_out, void* v_out,
                                       int cap_out, void* workspace, size_t ws_bytes,
                                       hipStream_t stream, Trace* tr) {
  if (dt != KVSEL_BF16 && dt != KVSEL_F32) return KVSEL_ERR_INVALID_ARG;
  kvsel_status st = check_cut_common(lengths, b, hq, hkv, cap, n_sink, T, kept_len_out);
  if (st != KVSEL_OK) return st;
  if (layer < 0 || n_full_layers < 0 || k_rows < 1 || k_rows > cap) return KVSEL_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return KVSEL_ERR_UNSUPPORTED;
  if (k_out) {
    if (!k || !v || !v_out || cap_out < cap) return KVSEL_ERR_INVALID_ARG;
    if (!aligned16(v) || !aligned16(k_out) || !aligned16(v_out)) return KVSEL_ERR_INVALID_ARG;
  }
  const int g = hq / hkv;
  const int grp = cut_group_rows(g, k_rows);
  const CutWs need = cut_ws(nullptr, b, hkv, grp, cap);
  if (!workspace || ws_bytes < need.bytes) return KVSEL_ERR_WORKSPACE;
  const CutWs ws = cut_ws(workspace, b, hkv, grp, cap);
  CutParams c = cut_params(ws, lengths, b, hq, hkv, cap, n_sink, T, kept_len_out);
  if (layer < n_full_layers) {
    KV_TRY(launch_cut_full(c, stream, tr));
  } else {
    if (!q_rows || !k || !aligned16(q_rows) || !aligned16(k)) return KVSEL_ERR_INVALID_ARG;
    ScoreParams p{};
    p.q = static_cast<const char*>(q_rows);
    p.k = static_cast<const char*>(k);
    p.lengths = lengths;
    p.b = b;
    p.hq = hq;
    p.hkv = hkv;
    p.g = g;
    p.w = k_rows;
    p.krows = k_rows;
    p.cap = cap;
    p.nchunk = c.nchunk;
    p.scale2 = kLog2e / sqrtf((float)d);
    p.cstat = ws.cstat;
    p.rstat = ws.rstat;
    p.logits = ws.logits;  // null: energies from recomputed logits
    p.energy = ws.energy;
    p.ctot = ws.ctot;
    p.err = ws.err;
    c.logits = ws.logits;
    c.attn = nullptr;
    // the g*k_rows rows of a KV head in groups of at most kMaxRows; each group
    // adds its rows' integer energy terms to the earlier groups'
    const int rows = g * k_rows;
    for (int r0 = 0; r0 < rows; r0 += grp) {
      p.rows0 = r0;
      p.m = rows - r0 < grp ? rows - r0 : grp;
      p.mp = rows_padded(p.m);
      KV_TRY(launch_stats(dt, d, kModeCut, p, stream, tr));
      KV_TRY(launch_reduce(d, kModeCut, p, stream, tr));
      if (ws.logits) {
        c.rows = p.m;
        c.mp = p.mp;
        c.accum = r0 > 0;
        KV_TRY(launch_cut_energy(c, stream, tr));
      } else {
        p.accum = r0 > 0;
        KV_TRY(launch_pool(dt, d, kModeCut, p, stream, tr));
      }
    }
    KV_TRY(launch_cut_scan(c, stream, tr));
  }
  if (k_out) {
    CutCompactParams cp{static_cast<const char*>(k), static_cast<const char*>(v),
                        static_cast<char*>(k_out), static_cast<char*>(v_out), lengths,
                        kept_len_out, b, hkv, cap, cap_out, n_sink};
    KV_TRY(launch_cut_compact(dt, d, cp, stream, tr));
  }
  return KVSEL_OK;
}

kvsel_status kvsel_threshold_cut(kvsel_dtype dt, const void* q_last, const void* k,
                                 const int32_t* lengths, int b, int hq, int hkv, int d, int cap,
                                 int layer, int n_full_layers, int n_sink, float T,
                                 int32_t* kept_len_out, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
  return threshold_cut_impl(dt, q_last, 1, k, nullptr, lengths, b, hq, hkv, d, cap, layer,
                            n_full_layers, n_sink, T, kept_len_out, nullptr, nullptr, 0,
                            workspace, ws_bytes, stream, nullptr);
}

kvsel_status kvsel_threshold_cut_rows(kvsel_dtype dt, const void* q_rows, int k_rows,
                                      const void* k, const void* v, const int32_t* lengths, int b,
                                      int hq, int hkv, int d, int cap, int layer,
                                      int n_full_layers, int n_sink, float T,
                                      int32_t* kept_len_out, void* k_out, void* v_out,
                                      int cap_out, void* workspace, size_t ws_bytes,
                                      hipStream_t stream) {
  return threshold_cut_impl(dt, q_rows, k_rows, k, v, lengths, b, hq, hkv, d, cap, layer,
                            n_full_layers, n_sink, T, kept_len_out, k_out, v_out, cap_out,
                            workspace, ws_bytes, stream, nullptr);
}

kvsel_status kvsel_threshold_cut_rows_traced(kvsel_dtype dt, const void* q_rows, int k_rows,
                                             const void* k, const void* v,
                                             const int32_t* lengths, int b, int hq, int hkv,
                                             int d, int cap, int layer, int n_full_layers,
                                             int n_sink, float T, int32_t* kept_len_out,
                                             void* k_out, void* v_out, int cap_out,
                                             void* workspace, size_t ws_bytes,
                                             hipStream_t stream, hipEvent_t* events,
                                             int n_events) {
  if (!events || n_events < 2) return KVSEL_ERR_INVALID_ARG;
  Trace tr{events, n_events, 0};
  return threshold_cut_impl(dt, q_rows, k_rows, k, v, lengths, b, hq, hkv, d, cap, layer,
                            n_full_layers, n_sink, T, kept_len_out, k_out, v_out, cap_out,
                            workspace, ws_bytes, stream, &tr);
}

kvsel_status kvsel_cut_compact(kvsel_dtype dt, const void* k, const void* v,
                               const int32_t* lengths, const int32_t* kept_len, int b, int hkv,
                               int d, int cap, int n_sink, void* k_out, void* v_out, int cap_out,
                               hipStream_t stream) {
  if (dt != KVSEL_BF16 && dt != KVSEL_F32) return KVSEL_ERR_INVALID_ARG;
  if (!k || !v || !lengths || !kept_len || !k_out || !v_out) return KVSEL_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out))
    return KVSEL_ERR_INVALID_ARG;
  if (b < 1 || hkv < 1 || cap < 1 || n_sink < 0 || cap_out < 1) return KVSEL_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return KVSEL_ERR_UNSUPPORTED;
  if (b > 65535 || hkv > 65535 || cap >= (1 << 24)) return KVSEL_ERR_UNSUPPORTED;
  CutCompactParams cp{static_cast<const char*>(k), static_cast<const char*>(v),
                      static_cast<char*>(k_out), static_cast<char*>(v_out), lengths, kept_len, b,
                      hkv, cap, cap_out, n_sink};
  return hip_status(launch_cut_compact(dt, d, cp, stream, nullptr));
}

kvsel_status kvsel_threshold_cut_traced(kvsel_dtype dt, const void* q_last, const void* k,
                                        const int32_t* lengths, int b, int hq, int hkv, int d,
                                        int cap, int layer, int n_full_layers, int n_sink, float T,
                                        int32_t* kept_len_out, void* workspace, size_t ws_bytes,
                                        hipStream_t stream, hipEvent_t* events, int n_events) {
  if (!events || n_events < 2) return KVSEL_ERR_INVALID_ARG;
  Trace tr{events, n_events, 0};
  return threshold_cut_impl(dt, q_last, 1, k, nullptr, lengths, b, hq, hkv, d, cap, layer,
                            n_full_layers, n_sink, T, kept_len_out, nullptr, nullptr, 0,
                            workspace, ws_bytes, stream, &tr);
}

kvsel_status kvsel_threshold_cut_from_attn(const float* attn_last, const int32_t* lengths, int b,
                                           int hq, int hkv, int cap, int n_sink, float T,
                                           int32_t* kept_len_out, void* workspace,
                                           size_t ws_bytes, hipStream_t stream) {
  kvsel_status st = check_cut_common(lengths, b, hq, hkv, cap, n_sink, T, kept_len_out);
  if (st != KVSEL_OK) return st;
  if (!attn_last) return KVSEL_ERR_INVALID_ARG;
  const int g = hq / hkv;
  const CutWs need = cut_ws(nullptr, b, hkv, g, cap);
  if (!workspace || ws_bytes < need.bytes) return KVSEL_ERR_WORKSPACE;
  const CutWs ws = cut_ws(workspace, b, hkv, g, cap);
  CutParams c = cut_params(ws, lengths, b, hq, hkv, cap, n_sink, T, kept_len_out);
  c.attn = attn_last;
  c.logits = nullptr;
  KV_TRY(launch_cut_energy(c, stream, nullptr));
  KV_TRY(launch_cut_scan(c, stream, nullptr));
  return KVSEL_OK;
}

kvsel_status kvsel_workspace_error(const void* workspace, int32_t* flags_host, hipStream_t stream) {
  if (!workspace || !flags_host) return KVSEL_ERR_INVALID_ARG;
  KV_TRY(hipMemcpyAsync(flags_host, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  KV_TRY(hipStreamSynchronize(stream));
  return KVSEL_OK;
}

}  // extern "C"
