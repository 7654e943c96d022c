/*
 * kvsel.h — C ABI of libkvsel, the MI355X (gfx950) KV-cache score-and-evict
 * library.  Every entry point launches hand-written HIP kernels on the
 * caller's stream and returns without synchronising.
 *
 * Two selection rules:
 *
 *  R-KV (QbitAI R-KV article, section "R-KV三步走：冗余识别+重要性评估+动态淘汰"):
 *   per KV head h of sequence b, with n = lengths[b] cached tokens,
 *     importance  I[j] = mean over the g*w window rows (q, r) of the GQA group
 *                        of softmax_j(Q[q,r] . K[j] / sqrt(d))
 *     redundancy  R[j] = (1/(n-1)) * sum over i != j of cos(K[i], K[j])
 *                        (a zero key has cosine 0; R = 0 when n == 1)
 *     score       Z[j] = lambda * I[j] - (1 - lambda) * R[j]
 *     selection   the min(budget, n) largest Z, equal Z -> lower position,
 *                 written in ascending position order
 *     compaction  K_out[t] = K[idx[t]], V_out[t] = V[idx[t]] (bit copies).
 *   The article names the parts (attention-based importance, key-cosine
 *   redundancy, joint eviction under a KV budget, lambda about 0.1); the exact
 *   formulas above are the plain reading of it.
 *
 *  ReFreeKV (review "论文综述：ReFreeKV：迈向无阈值的KV缓存压缩", section 二, first
 *   and second step and the efficiency paragraph): per KV head, tokens are
 *   queued sinks first (positions 0..m-1) then newest to oldest; the energy of
 *   token j is e[j] = sum over the group's g last-row queries of a[q,j]^2 with
 *   a = softmax_j(q_last . K[j] / sqrt(d)); the kept length is
 *     L = max(min(m, n), smallest p >= 1 whose first p queued tokens hold
 *             >= (1 - T) of the total energy),
 *   layers below n_full_layers keep L = n.  Energies enter the walk as
 *   fixed-point integers (each fp32 square floored at 2^-52 resolution) so the
 *   walk itself is exact and independent of summation order.
 *
 * Layouts (all row-major, element type per kvsel_dtype):
 *   q_window [b][Hq][w][d], q_last [b][Hq][d],
 *   k, v     [b][Hkv][cap][d]        (token j of head h of sequence b at row j)
 *   lengths  [b] int32 on the device; a value outside [0, cap] is clamped into
 *            it (a negative length holds no tokens) and reported by
 *            kvsel_workspace_error().
 *   GQA: query head q belongs to KV head q / (Hq / Hkv).
 *
 * Ownership: the caller allocates every buffer, device workspace included;
 * the library allocates nothing and keeps no state between calls.  Inputs are
 * never written (kvsel_slots_write, which updates a cache in place, aside).
 * A workspace may serve one call at a time; calls that share one must be
 * ordered on one stream.  Every entry point only launches kernels on the
 * given stream (no memory sets, copies or synchronisation), so a call can be
 * captured into a HIP graph and replayed; kvsel_workspace_error reads back
 * and synchronises and is the exception.
 *
 * Errors: argument checks run on the host before any launch and return
 * KVSEL_ERR_INVALID_ARG / KVSEL_ERR_UNSUPPORTED / KVSEL_ERR_WORKSPACE with
 * nothing launched; a failed launch returns KVSEL_ERR_HIP.  Pointers are
 * device pointers unless stated otherwise.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVSEL_OK = 0,
  KVSEL_ERR_INVALID_ARG = 1,
  KVSEL_ERR_UNSUPPORTED = 2,
  KVSEL_ERR_WORKSPACE = 3,
  KVSEL_ERR_HIP = 4
} kvsel_status;

typedef enum { KVSEL_BF16 = 0, KVSEL_F32 = 1 } kvsel_dtype;

/* How R is evaluated.  Both give the same R up to fp32 rounding.
 *  KVSEL_R_GRAM:   the n x n Gram matrix K.K^T on bf16 matrix cores (fp32
 *                  accumulation), weighted by inverse norms and row-summed in
 *                  registers; the n x n matrix never reaches memory.  Each
 *                  pair of 256-key blocks is computed once (symmetry), about
 *                  n^2 d multiply-adds.  O(n^2 d).
 *  KVSEL_R_KEYSUM: the regrouped sum  sum_{i!=j} u_i.u_j = u_j.(sum_i u_i) - u_j.u_j
 *                  over unit keys u, fused into the importance pass.  O(n d). */
typedef enum { KVSEL_R_GRAM = 0, KVSEL_R_KEYSUM = 1 } kvsel_redundancy;

/* Supported: d in {64, 128}; g*w <= 128 (R-KV); g <= 32 (ReFreeKV);
 * 1 <= budget <= 65536; cap <= 2^24 - 1. */

const char* kvsel_status_string(kvsel_status s);

/* ---------------------------------------------------------------- R-KV */

/* Bytes of device workspace kvsel_scores / kvsel_score_evict need. */
size_t kvsel_score_evict_workspace(int b, int Hq, int Hkv, int d, int w, int cap, int budget);

/* Scores only.  Writes Z (and I, R when non-null) as fp32 [b][Hkv][cap];
 * entries at positions >= n are left untouched.  lambda in [0, 1].
 * Key-sum form on a cache of more than 4096 slots (bf16, d = 128, g*w <= 32):
 * when the grid of ceil(cap / 256) * Hkv * b work-groups fits on the device
 * at once (1024 on 256 compute units), one kernel computes the scores,
 * reading each key once; otherwise, or with KVSEL_SEPARATE_KERNELS=1 in the
 * environment, the
 * statistics, their merge and the pooling run as separate kernels.  Both give
 * the same bits.  The one-launch kernels (this one and the short-cache step
 * of kvsel_score_evict) wait on work-groups of the same head: kernels of
 * other streams that hold compute units for milliseconds can make a wait
 * run out (reported in bit 2 of the error word); KVSEL_SEPARATE_KERNELS=1
 * avoids them. */
kvsel_status kvsel_scores(kvsel_dtype dt, kvsel_redundancy mode,
                          const void* q_window, const void* k, const int32_t* lengths,
                          int b, int Hq, int Hkv, int d, int w, int cap, float lambda,
                          float* i_out, float* r_out, float* z_out,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/* Top-budget choice from given scores z [b][Hkv][cap] (fp32).  idx_out
 * [b][Hkv][budget] int32 receives the positions of the min(budget, n) largest
 * scores (equal scores: lower position first) in ascending order, then -1.
 * -0.0 is treated as +0.0; z must hold no NaN.  Needs a device workspace of
 * kvsel_select_workspace() bytes. */
size_t kvsel_select_workspace(int b, int Hkv, int cap);
kvsel_status kvsel_select_topb(const float* z, const int32_t* lengths, int b, int Hkv,
                               int cap, int budget, int32_t* idx_out,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/* Top-budget choice with one budget per KV head: head h keeps the
 * min(budgets[h], n) largest scores, chosen and ordered as in
 * kvsel_select_topb.  budgets [Hkv] int32 on the device is one row of a
 * static per-(layer, head) budget table: the LU-KV page (Baidu Baige and
 * Fudan, "Predicting Future Utility"), third step, profiles the best budget
 * share of every head offline into a lookup table and reads it at inference
 * time before the per-head eviction runs; that table's row is this argument.
 * idx_out is [b][Hkv][budget_max]: head h's entries, then -1 up to
 * budget_max.  A budget outside [0, budget_max] is clamped into it and sets
 * bit 1 of the workspace error word; budget 0 keeps nothing.  Same workspace
 * size as kvsel_select_topb. */
kvsel_status kvsel_select_topb_heads(const float* z, const int32_t* lengths,
                                     const int32_t* budgets, int b, int Hkv, int cap,
                                     int budget_max, int32_t* idx_out,
                                     void* workspace, size_t ws_bytes, hipStream_t stream);

/* Gather-compaction: for t < budget with idx[t] >= 0, row t of k_out/v_out
 * [b][Hkv][cap_out][d] becomes row idx[t] of k/v (bit copy); other rows are
 * left untouched.  idx values must lie in [0, cap) or be -1. */
kvsel_status kvsel_gather(kvsel_dtype dt, const void* k, const void* v, const int32_t* idx,
                          int b, int Hkv, int d, int cap, int budget,
                          void* k_out, void* v_out, int cap_out, hipStream_t stream);

/* The whole step: scores, top-budget, gather.  budget <= cap_out.
 * scores_out (nullable) receives Z as in kvsel_scores.  A short cache with
 * the key-sum form (bf16, d = 128, g*w <= 32, cap <= 4096) runs as a single
 * launch when its grid of ceil(cap / 256) * Hkv * b work-groups fits on the
 * device at once (the device's capacity for that kernel is queried once per
 * device and kept); its scores and selection are identical to the
 * multi-kernel path's. */
kvsel_status kvsel_score_evict(kvsel_dtype dt, kvsel_redundancy mode,
                               const void* q_window, const void* k, const void* v,
                               const int32_t* lengths, int b, int Hq, int Hkv, int d, int w,
                               int cap, float lambda, int budget,
                               void* k_out, void* v_out, int cap_out,
                               int32_t* idx_out, float* scores_out,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/* Bytes of the device array kvsel_score_evict_static works in (16 MiB per
 * GPU the library runs on, held until the process ends). */
#define KVSEL_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

/* kvsel_score_evict without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The call works in a file-scope device
 * array of KVSEL_STATIC_SCRATCH_BYTES (one per GPU) and allocates nothing;
 * the caller still passes every input and output.  Same arguments, results
 * and error returns as kvsel_score_evict, plus KVSEL_ERR_WORKSPACE when the
 * call's layout exceeds the array: the key-sum form needs about
 * 11 bytes per (sequence, KV head, cap position) (2.9 MiB at 8 KV heads and
 * cap 32768); the Gram form about 12 + 4 * ceil(cap / 256) / 2 bytes per
 * position (1.5 MiB at 8 KV heads and cap 2176; caps above about 8192 at
 * 8 heads do not fit).  Calls share the array: every call overwrites it, and
 * calls that overlap on one GPU (on different streams, or from several
 * threads without ordering) race.  Lengths outside [0, cap] are clamped as
 * in kvsel_score_evict but not reported (kvsel_workspace_error needs a
 * workspace). */
kvsel_status kvsel_score_evict_static(kvsel_dtype dt, kvsel_redundancy mode,
                                      const void* q_window, const void* k, const void* v,
                                      const int32_t* lengths, int b, int Hq, int Hkv, int d, int w,
                                      int cap, float lambda, int budget,
                                      void* k_out, void* v_out, int cap_out,
                                      int32_t* idx_out, float* scores_out, hipStream_t stream);

/* The whole step with one budget per KV head (budgets [Hkv] int32 on the
 * device, as in kvsel_select_topb_heads): k_out/v_out [b][Hkv][cap_out][d]
 * receive head h's kept rows in rows 0 .. min(budgets[h], n)-1, later rows
 * are left untouched; idx_out is [b][Hkv][budget_max] with -1 padding.
 * budget_max <= cap_out.  Same workspace size as kvsel_score_evict. */
kvsel_status kvsel_score_evict_heads(kvsel_dtype dt, kvsel_redundancy mode,
                                     const void* q_window, const void* k, const void* v,
                                     const int32_t* lengths, const int32_t* budgets,
                                     int b, int Hq, int Hkv, int d, int w, int cap, float lambda,
                                     int budget_max, void* k_out, void* v_out, int cap_out,
                                     int32_t* idx_out, float* scores_out,
                                     void* workspace, size_t ws_bytes, hipStream_t stream);

/* Same step with per-kernel timing for profilers and benchmarks: kernel k of
 * the call records events[2k] when it starts and events[2k+1] when it ends
 * (k < n_events / 2; events are created by the caller with hipEventCreate).
 * Launch order for cap <= 32768: KVSEL_R_GRAM: stats, reduce, pool, gram,
 * gram_fin, threshold, compact (the compaction kernel also gathers the kept rows);
 * KVSEL_R_KEYSUM: stats, reduce, pool, threshold, compact.  For larger cap
 * the last two are replaced by select, gather.  With cap <= 4096 (at most 16
 * chunks of 256 keys per head) there is no reduce kernel: pool merges the
 * chunk partials itself; a key-sum call that takes the single-launch path
 * (see kvsel_score_evict) launches one kernel, and one that takes the
 * one-launch score pass (see kvsel_scores) launches scores, threshold,
 * compact (select, gather above cap 32768).  Threshold and compact become
 * one kernel, select_compact, when a chunk of 512 positions keeps about 64
 * rows or fewer (budget <= cap / 8), fewer than 64 heads are scored and the
 * whole grid fits on the device at once (each work-group finds the threshold
 * from every chunk's published candidates and compacts its own chunk: the
 * same bits; KVSEL_SEPARATE_KERNELS=1 keeps the two kernels). */
kvsel_status kvsel_score_evict_traced(kvsel_dtype dt, kvsel_redundancy mode,
                                      const void* q_window, const void* k, const void* v,
                                      const int32_t* lengths, int b, int Hq, int Hkv, int d,
                                      int w, int cap, float lambda, int budget,
                                      void* k_out, void* v_out, int cap_out,
                                      int32_t* idx_out, float* scores_out,
                                      void* workspace, size_t ws_bytes, hipStream_t stream,
                                      hipEvent_t* events, int n_events);

/* kvsel_score_evict_heads with per-kernel timing as in kvsel_score_evict_traced. */
kvsel_status kvsel_score_evict_heads_traced(kvsel_dtype dt, kvsel_redundancy mode,
                                            const void* q_window, const void* k, const void* v,
                                            const int32_t* lengths, const int32_t* budgets,
                                            int b, int Hq, int Hkv, int d, int w, int cap,
                                            float lambda, int budget_max, void* k_out,
                                            void* v_out, int cap_out, int32_t* idx_out,
                                            float* scores_out, void* workspace, size_t ws_bytes,
                                            hipStream_t stream, hipEvent_t* events, int n_events);

/* ---------------------------------------------------------- slot reuse */

/* Gather-free eviction for a cache that is never compacted (ThinKV page,
 * "Continuous Thinking" section: compaction by gather rewrites the cache on
 * every eviction, which evicted-slot reuse avoids).  Slots 0..n-1 of each
 * (sequence, KV head) all hold tokens; pos [b][Hkv][cap] int32 (nullable:
 * the slot index) holds the token position in each slot, non-negative and
 * distinct per head.  The kept set is the min(B_h, n) largest scores, equal
 * scores going to the lower token position (equal positions: lower slot), as
 * in kvsel_select_topb; B_h is budget, or budgets[h] clamped to [0, budget]
 * when budgets (nullable, [Hkv]) is given.  evict_out [b][Hkv][evict_stride]
 * receives the other n - min(B_h, n) slots in ascending slot order, then -1;
 * n_evict_out [b][Hkv] their count.  evict_stride >= cap - budget (>= cap
 * with budgets).  Needs cap <= 32768.  Same workspace size as
 * kvsel_select_topb. */
kvsel_status kvsel_select_evict_slots(const float* z, const int32_t* lengths, const int32_t* pos,
                                      const int32_t* budgets, int b, int Hkv, int cap, int budget,
                                      int32_t* evict_out, int evict_stride, int32_t* n_evict_out,
                                      void* workspace, size_t ws_bytes, hipStream_t stream);

/* Scores (as kvsel_scores) then kvsel_select_evict_slots in one call; k is
 * read only.  Same workspace size as kvsel_score_evict.  Key-sum form on a
 * cache of at most 4096 slots (bf16, d = 128, g*w <= 32), when its grid of
 * ceil(cap / 256) * Hkv * b work-groups fits on the device at once: one
 * kernel computes the scores, the threshold and the evicted list (the same
 * scores and the same list as the separate kernels, which run otherwise or
 * with KVSEL_SEPARATE_KERNELS=1).  Gram form on such caches (cap <= 4096):
 * after the score kernels up to the Gram units, one kernel forms Z, the
 * threshold and the evicted list, under the same conditions. */
kvsel_status kvsel_score_evict_slots(kvsel_dtype dt, kvsel_redundancy mode,
                                     const void* q_window, const void* k, const int32_t* lengths,
                                     const int32_t* pos, const int32_t* budgets,
                                     int b, int Hq, int Hkv, int d, int w, int cap, float lambda,
                                     int budget, int32_t* evict_out, int evict_stride,
                                     int32_t* n_evict_out, float* scores_out,
                                     void* workspace, size_t ws_bytes, hipStream_t stream);

/* kvsel_score_evict_slots with per-kernel timing as in kvsel_score_evict_traced.
 * Launch order: the score kernels of the mode, threshold, evict; or the
 * single kernel of the short-cache key-sum form. */
kvsel_status kvsel_score_evict_slots_traced(kvsel_dtype dt, kvsel_redundancy mode,
                                            const void* q_window, const void* k,
                                            const int32_t* lengths, const int32_t* pos,
                                            const int32_t* budgets, int b, int Hq, int Hkv, int d,
                                            int w, int cap, float lambda, int budget,
                                            int32_t* evict_out, int evict_stride,
                                            int32_t* n_evict_out, float* scores_out,
                                            void* workspace, size_t ws_bytes, hipStream_t stream,
                                            hipEvent_t* events, int n_events);

/* New tokens into evicted slots: for each (sequence, KV head), token t <
 * min(count, n_evict[b][h]) of k_new/v_new [b][Hkv][count][d] is copied (bit
 * copy) into slot evict[b][h][t] of k/v [b][Hkv][cap][d], and, when pos is
 * given, pos[b][h][slot] = pos_new[b] + t (pos_new [b] required then).
 * Tokens beyond the evicted count are not written; evict entries outside
 * [0, cap) are skipped. */
kvsel_status kvsel_slots_write(kvsel_dtype dt, void* k, void* v, int32_t* pos,
                               const void* k_new, const void* v_new, const int32_t* pos_new,
                               const int32_t* evict, int evict_stride, const int32_t* n_evict,
                               int b, int Hkv, int d, int cap, int count, hipStream_t stream);

/* ------------------------------------------------------------ ReFreeKV */

size_t kvsel_threshold_cut_workspace(int b, int Hq, int Hkv, int d, int cap);

/* Kept length per (sequence, KV head) into kept_len_out [b][Hkv] int32.
 * layer < n_full_layers: L = n without reading K.  n_sink >= 0, T in [0, 1). */
kvsel_status kvsel_threshold_cut(kvsel_dtype dt, const void* q_last, const void* k,
                                 const int32_t* lengths, int b, int Hq, int Hkv, int d, int cap,
                                 int layer, int n_full_layers, int n_sink, float T,
                                 int32_t* kept_len_out,
                                 void* workspace, size_t ws_bytes, hipStream_t stream);

/* kvsel_threshold_cut with per-kernel timing as in kvsel_score_evict_traced.
 * Launch order: stats, reduce, energy, scan (layer >= n_full_layers) or a
 * single fill kernel (layer < n_full_layers). */
kvsel_status kvsel_threshold_cut_traced(kvsel_dtype dt, const void* q_last, const void* k,
                                        const int32_t* lengths, int b, int Hq, int Hkv, int d,
                                        int cap, int layer, int n_full_layers, int n_sink, float T,
                                        int32_t* kept_len_out, void* workspace, size_t ws_bytes,
                                        hipStream_t stream, hipEvent_t* events, int n_events);

/* The cut from the last k_rows attention rows instead of the single last row
 * (the review's ablation of its k = 1 simplification, e.g. k = 10% of n; same
 * section, ablation paragraph), optionally followed by the sink + suffix
 * compaction.  q_rows [b][Hq][k_rows][d]: row r of a query head is the query
 * of token n_b - k_rows + r and sees keys j <= n_b - k_rows + r (causal);
 * rows of tokens before position 0 contribute nothing.  The energy of token j
 * is the sum over the g*k_rows rows of the group of floor(fl32(a*a) * 2^52),
 * then the same walk and cut as kvsel_threshold_cut; k_rows = 1 gives
 * exactly kvsel_threshold_cut.  1 <= k_rows <= cap; the rows are scored in
 * groups of 128, so the cost grows as k_rows * n.  When a group has at most
 * 32 rows the scoring pass stores their logits in the workspace and the
 * energy pass reads them back; larger groups store none, and the energy pass
 * recomputes the logits from Q and K on the matrix cores (one more read of K
 * per group) and forms a^2 * 2^20 as a single power of two, so its terms may
 * differ from the stored-logit form in the last bits of a^2.  When k_out is non-null,
 * k_out/v_out [b][Hkv][cap_out][d] (cap_out >= cap) receive the kept tokens
 * in position order: the min(n_sink, n) sinks, then the newest L - sinks
 * (bit copies); rows from L on are left untouched.  Workspace:
 * kvsel_threshold_cut_rows_workspace. */
size_t kvsel_threshold_cut_rows_workspace(int b, int Hq, int Hkv, int d, int cap, int k_rows);
kvsel_status kvsel_threshold_cut_rows(kvsel_dtype dt, const void* q_rows, int k_rows,
                                      const void* k, const void* v, const int32_t* lengths,
                                      int b, int Hq, int Hkv, int d, int cap, int layer,
                                      int n_full_layers, int n_sink, float T,
                                      int32_t* kept_len_out, void* k_out, void* v_out,
                                      int cap_out, void* workspace, size_t ws_bytes,
                                      hipStream_t stream);

/* kvsel_threshold_cut_rows with per-kernel timing as in kvsel_score_evict_traced.
 * Launch order: stats, reduce, energy once per group of 128 rows, then scan,
 * then compact when k_out is given (a fill kernel replaces the scoring
 * kernels for layer < n_full_layers). */
kvsel_status kvsel_threshold_cut_rows_traced(kvsel_dtype dt, const void* q_rows, int k_rows,
                                             const void* k, const void* v,
                                             const int32_t* lengths, int b, int Hq, int Hkv,
                                             int d, int cap, int layer, int n_full_layers,
                                             int n_sink, float T, int32_t* kept_len_out,
                                             void* k_out, void* v_out, int cap_out,
                                             void* workspace, size_t ws_bytes,
                                             hipStream_t stream, hipEvent_t* events,
                                             int n_events);

/* Stage entry: the sink + suffix compaction from given kept lengths
 * kept_len [b][Hkv] (device): row t < L of k_out/v_out [b][Hkv][cap_out][d]
 * is position t for t < min(n_sink, n), else position n - L + t; rows from
 * min(L, cap_out) on are left untouched. */
kvsel_status kvsel_cut_compact(kvsel_dtype dt, const void* k, const void* v,
                               const int32_t* lengths, const int32_t* kept_len, int b, int Hkv,
                               int d, int cap, int n_sink, void* k_out, void* v_out, int cap_out,
                               hipStream_t stream);

/* Stage entry: the same cut from given fp32 last-row attention probabilities
 * attn_last [b][Hq][cap] (values in [0, 1], used as given; squares are
 * clamped to 1).  Same workspace size as kvsel_threshold_cut. */
kvsel_status kvsel_threshold_cut_from_attn(const float* attn_last, const int32_t* lengths,
                                           int b, int Hq, int Hkv, int cap, int n_sink, float T,
                                           int32_t* kept_len_out,
                                           void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ utility */

/* Reads the device error word left in the workspace by the last call that
 * used it (synchronises the stream).  Bit 0: some lengths[i] lay outside
 * [0, cap] and was clamped into it; bit 1: some per-head budget lay outside
 * [0, budget_max] and was clamped; bit 2: a wait between the work-groups of
 * the single-launch short-cache step, of the one-launch score pass or of
 * the one-launch selection exceeded its poll limit (the results of that call are not to be trusted;
 * it cannot happen while the device runs the whole grid at once, which the
 * library checks before choosing those paths, unless kernels of other
 * streams hold compute units for that long); bit 3: a work-group of the
 * single-launch short-cache step found a threshold that does not keep
 * exactly the budget, which a consistent selection never does (that
 * work-group writes no slots or rows; the call's results are not to be
 * trusted).  Returns KVSEL_ERR_HIP if the copy
 * fails. */
kvsel_status kvsel_workspace_error(const void* workspace, int32_t* flags_host, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVSEL_H */
