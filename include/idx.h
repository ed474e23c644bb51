/* Causal lightning-indexer library for AMD Instinct MI355X (gfx950): C ABI.
 *
 * What the library computes (cited by page title and section):
 *
 *  - "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention",
 *    Abstract: the indexer of token-level sparse attention scores every
 *    preceding token of each query and keeps a per-query top-k; PIVOT groups
 *    nearby queries, aggregates each group into one proxy query, runs one
 *    shared full-prefix scan to a candidate set, then either re-scores the
 *    candidates with each member's own indexer and keeps each member's own
 *    top-k (Refine) or shares the proxy's top-k with the group (Reuse).
 *    Groups are fixed-size runs of consecutive queries in prefill and the
 *    queries of one multi-token-prediction step in decode.
 *  - "ADIndex Restructures Sparse-Attention Indexing with Group-Level
 *    Distillation", "Why the Indexer Becomes the Bottleneck": in prefill all
 *    queries re-scan the same prefix; in decode each new query scans the
 *    whole cached key history.  "Deployment Guidance": the full scan is kept
 *    as the fallback path (idx_score_topk).
 *  - "MLI Restructures DeepSeek Sparse Attention ...", "Core Idea": the
 *    indexer keeps k = 2048 positions per query.
 *
 * Score (no page prints it; the DeepSeek lightning-indexer form is the
 * reading):  I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]),  s <= pos(t),
 * with pos(t) = q_pos0 + t.  For FP8 storage the real values are
 * code * per-token scale.  Top-k order: score descending, then key index
 * ascending (exact equality is a tie; -0 equals +0).  Rows with fewer
 * eligible keys than k are filled with all of them and padded with -1.
 * Each output row is a set: the order of its entries is unspecified.
 *
 * Conventions for every entry point:
 *  - Pointers named q, k, w, scales, out_*, cand, proxy_topk and ws are DEVICE
 *    pointers to contiguous row-major buffers owned by the caller; the
 *    idx_problem struct itself is a HOST pointer.  The library never
 *    allocates or frees device memory and never synchronizes: all work is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *  - Errors: every check is made on the host before anything is enqueued,
 *    and on error nothing is enqueued.  IDX_EINVAL: a null required pointer,
 *    a non-positive size, q_pos0 < 0 or q_pos0 + n_q > n_k, topk/group/n_cand
 *    < 1, a scale pointer present for non-FP8 storage or missing for FP8.
 *    IDX_EUNSUPPORTED: a (heads, dim, q dtype, k dtype) combination without a
 *    kernel (supported: heads in {16, 32, 64}, dim in {64, 128}; dtypes
 *    (F32, F32), (BF16, BF16), (BF16, FP8_E4M3), (FP8_E4M3, FP8_E4M3)).
 *    IDX_EWORKSPACE: ws_bytes smaller than idx_workspace_bytes() reports as
 *    the minimum.  IDX_EHIP: a HIP launch error (hipGetLastError).
 *    Device-side faults surface at the caller's next synchronization; after
 *    any error the outputs are undefined.
 *  - Preconditions that are not checked: finite inputs, scales > 0, no
 *    aliasing between outputs and inputs, n_k < 2^31.  Calls on distinct
 *    workspaces are independent; two calls that share a workspace must be
 *    ordered on one stream.
 *  - HIP graph capture: a call may be captured on `stream` once the same
 *    call shape (dtypes, heads, dim, mode) has run once uncaptured on the
 *    device, since the first launch of some kernels sets their LDS limit
 *    (hipFuncSetAttribute).  Capture with profiling off (idx_profile_enable).
 */
#ifndef SATC_IDX_H
#define SATC_IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats.  IDX_FP8_E4M3 is the OCP FP8 E4M3 format ("e4m3fn":
 * bias 7, no infinities, max 448) with one float32 scale per token. */
enum { IDX_F32 = 0, IDX_BF16 = 1, IDX_FP8_E4M3 = 2 };

enum {
  IDX_OK = 0,
  IDX_EINVAL = -1,
  IDX_EUNSUPPORTED = -2,
  IDX_EWORKSPACE = -3,
  IDX_EHIP = -4,
  IDX_ETOOLARGE = -5  /* beyond the fixed scratch of idx_score_topk_static */
};

/* Operation codes for idx_workspace_bytes. */
enum {
  IDX_OP_SCORE_TOPK = 0,
  IDX_OP_GROUP_PROXY_SCAN = 1,
  IDX_OP_REFINE_TOPK = 2,
  IDX_OP_REUSE_TOPK = 3,
  IDX_OP_BLOCK_ROUTE = 4, /* n_cand = block size, topk = blocks kept */
  IDX_OP_IVF_BUILD = 5,   /* n_cand = clusters per version; only the key fields of p are read */
  IDX_OP_IVF_ROUTE = 6    /* group, n_cand = clusters per version */
};

/* One indexer problem: B sequences, each with n_q queries and n_k keys.
 *   q       [B, n_q, heads, dim]  q_dtype   (dim fastest)
 *   q_scale [B, n_q] float32, per query token (FP8 q only, else NULL)
 *   k       [B, n_k, dim]         k_dtype
 *   k_scale [B, n_k] float32, per key token (FP8 k only, else NULL)
 *   w       [B, n_q, heads] float32 head weights
 * Query t of a sequence sits at position pos(t) = q_pos0 + t of its key
 * sequence: q_pos0 = 0 in prefill (n_q = n_k), n_k - n_q in decode (the key
 * cache already holds the new tokens' keys). */
typedef struct {
  int32_t batch, n_q, n_k, q_pos0, heads, dim;
  int32_t q_dtype, k_dtype;
  const void* q;
  const float* q_scale;
  const void* k;
  const float* k_scale;
  const float* w;
} idx_problem;

/* Library version (major*10000 + minor*100 + patch). */
int32_t idx_version(void);

/* Human-readable name of a status code (static storage; never NULL). */
const char* idx_status_string(int32_t status);

/* Workspace size in bytes that the operation `op` needs for problem `p`
 * (group/n_cand/topk as the call will pass them; ignored where unused).
 * Returns 0 when the operation needs none (or on invalid arguments).  Passing
 * a larger workspace is allowed. */
size_t idx_workspace_bytes(const idx_problem* p, int32_t op, int32_t group,
                           int32_t n_cand, int32_t topk);

/* Dense causal indexer ("full-scan" path; PIVOT, Abstract: score every
 * preceding token and keep each query's top-k).
 *   out_idx    [B, n_q, topk] int32: the top min(topk, pos(t)+1) key
 *              indices of each query, padded with -1.
 *   out_scores optional [B, n_q, n_k] float32: the exact scores the select
 *              used; positions beyond pos(t) are -inf.  NULL in timed runs.
 * ws/ws_bytes: workspace of at least idx_workspace_bytes(p, IDX_OP_SCORE_TOPK,
 * 0, 0, topk) bytes (may be NULL when that is 0). */
int32_t idx_score_topk(const idx_problem* p, int32_t topk, int32_t* out_idx,
                       float* out_scores, void* ws, size_t ws_bytes, void* stream);

/* idx_score_topk without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * (the decode step), harnesses that forbid allocation.  Same computation,
 * arguments, layouts and errors as idx_score_topk; its scratch is a fixed
 * device array of IDX_STATIC_SCRATCH_BYTES (64 MiB) that each GPU the library
 * runs on holds until the process ends (its address is resolved on the first
 * call on a device).  Returns IDX_ETOOLARGE, before enqueueing anything, when
 * idx_workspace_bytes(p, IDX_OP_SCORE_TOPK, 0, 0, topk) exceeds that size
 * (decode shapes fit: 8 sequences x 2 queries x 131072 keys need about
 * 41 MiB).  Calls no allocating routine.  Every call on one GPU shares the
 * array, which keeps the last call's contents (nothing in it needs to start
 * at zero): calls that overlap in time on one GPU - on different streams or
 * from different host threads without ordering - race and corrupt each
 * other's results; order them on one stream. */
#define IDX_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int32_t idx_score_topk_static(const idx_problem* p, int32_t topk, int32_t* out_idx, float* out_scores,
                              void* stream);

/* PIVOT proxy and shared scan (PIVOT, Abstract: aggregate a group into one
 * proxy query and run one shared full-prefix scan to a candidate set).
 * Groups are runs of `group` consecutive queries of one sequence (the last
 * may be shorter); n_g = ceil(n_q / group).  The proxy is the mean of the
 * members' real q and of their w (float32 arithmetic), stored as bfloat16
 * (round to nearest even) for BF16/FP8 q and as float32 for F32 q; FP8 keys
 * are widened to bfloat16 (exactly) for the scan.  The scan of group g
 * covers keys 0..pos(last member of g).
 *   out_cand         [B, n_g, n_cand] int32: the top min(n_cand, prefix)
 *                    keys of the proxy, padded with -1.  With
 *                    n_cand = topk this is the Reuse input.
 *   out_proxy_q      optional [B, n_g, heads, dim] (bfloat16 or float32).
 *   out_proxy_w      optional [B, n_g, heads] float32.
 *   out_proxy_scores optional [B, n_g, n_k] float32, -inf beyond the prefix. */
int32_t idx_group_proxy_scan(const idx_problem* p, int32_t group, int32_t n_cand,
                             int32_t* out_cand, void* out_proxy_q, float* out_proxy_w,
                             float* out_proxy_scores, void* ws, size_t ws_bytes,
                             void* stream);

/* PIVOT-Refine (PIVOT, Abstract: re-score the candidate set with each
 * query's own indexer and select an individual top-k).  Member t of group g
 * considers V_t = { c in cand[b, g, :] : 0 <= c <= pos(t) } (entries outside
 * [0, n_k) are empty slots) and keeps its top min(topk, |V_t|).  Candidate
 * entries of one row must be distinct.
 *   cand            [B, n_g, n_cand] int32 (e.g. out_cand of the proxy scan).
 *   out_idx         [B, n_q, topk] int32, padded with -1.
 *   out_cand_scores optional [B, n_q, n_cand] float32, -inf for excluded slots. */
int32_t idx_refine_topk(const idx_problem* p, int32_t group, const int32_t* cand,
                        int32_t n_cand, int32_t topk, int32_t* out_idx,
                        float* out_cand_scores, void* ws, size_t ws_bytes,
                        void* stream);

/* PIVOT-Reuse (PIVOT, Abstract: share the proxy top-k across the group).
 * Member t of group g keeps { c in proxy_topk[b, g, :] : 0 <= c <= pos(t) }
 * in the proxy's order, padded with -1 (no refill).  Integer only; only
 * p->batch, n_q, n_k, q_pos0 are read (q/k/w may be NULL).
 *   proxy_topk [B, n_g, topk] int32, out_idx [B, n_q, topk] int32. */
int32_t idx_reuse_topk(const idx_problem* p, int32_t group, const int32_t* proxy_topk,
                       int32_t topk, int32_t* out_idx, void* stream);

/* Block-mean candidate routing, a second candidate generator for
 * idx_refine_topk ("AttentionIndex Architecture ...", "Why Positional Blocks
 * Lose Recall" and "Worked Example: Blocks Lose, Clusters Win": contiguous
 * blocks of keys are ranked by a mean-pooled representative, the best ones
 * are kept, and the native indexer then runs only on their keys).
 * Keys are cut into n_b = ceil(n_k / block) blocks of `block` consecutive
 * positions (the last may be shorter); block j is represented by the mean of
 * its real keys (float32 arithmetic, stored as bfloat16, or float32 for F32
 * keys).  Group g (as in idx_group_proxy_scan) routes with its proxy: block
 * j is routable iff all its keys lie in the prefix of the group's last
 * member, n_full(g) = floor((pos(t_last) + 1) / block) of them; the group
 * keeps the top min(n_sel, n_full(g)) routable blocks by
 * sum_h wbar[h] * max(0, qbar[h,:] . mean_j), ties to the lower block index.
 *   out_cand          [B, n_g, (n_sel + 1) * block] int32: the keys of the
 *                     kept blocks, then the keys of the trailing partial
 *                     block up to pos(t_last), padded with -1 (a candidate
 *                     row for idx_refine_topk with n_cand = its width; the
 *                     order within a row is unspecified).
 *   out_block_means   optional [B, n_b, dim] (bfloat16 or float32).
 *   out_block_scores  optional [B, n_g, n_b] float32, -inf where not routable.
 *   out_proxy_q/_w    optional, as in idx_group_proxy_scan.
 * ws: idx_workspace_bytes(p, IDX_OP_BLOCK_ROUTE, group, block, n_sel).
 * IDX_EINVAL also for block < 1, n_sel < 1, or a row width beyond 2^31 - 1. */
int32_t idx_block_route(const idx_problem* p, int32_t group, int32_t block, int32_t n_sel,
                        int32_t* out_cand, void* out_block_means, float* out_block_scores,
                        void* out_proxy_q, float* out_proxy_w, void* ws, size_t ws_bytes,
                        void* stream);

/* IVF index with causal versions, a third candidate generator for
 * idx_refine_topk ("AttentionIndex Architecture ...", "KEY FINDINGS" and "An
 * Inverted File With Causal Versions": keys are grouped by similarity into
 * inverted lists, a query is routed to the lists whose representatives score
 * highest and the native indexer re-scores their members; arriving keys
 * join existing lists batch by batch, and a refit now and then reclusters all
 * keys so far, seeded with the previous clustering, as a new version; a group
 * routes through a version only when all of that version's keys precede its
 * last member).  The
 * representatives here are plain means (no trained encoder).
 *
 * idx_ivf_build: for each sequence, versions u = 1 .. n_v = floor(n_k / R)
 * (R = refit).  Version u is refit on keys [0, u R) by `iters` Lloyd
 * iterations of k-means with m = n_clusters centroids, starting from version
 * u-1's centroids (version 1: the keys at positions floor(c R / m)).  An
 * iteration assigns each key to the nearest stored centroid (squared L2,
 * ties to the lower centroid) and replaces each centroid by the mean of its
 * members' real values (float32 sums; an empty cluster keeps its centroid).
 * Centroids are stored as bfloat16 (round to nearest even), float32 for F32
 * keys, and the stored values are what assignment and routing use.  The
 * published lists of version u hold every key of its window
 * [0, min((u + 1) R, n_k)) under its nearest centroid of version u, in key
 * order within each list.  Only p->batch, n_k, dim, k_dtype, k and k_scale
 * are read.  Outputs (n_tiles = ceil(n_k / 128)):
 *   out_centroids [B, n_v, m, dim]   bfloat16 (float32 for F32 keys)
 *   out_offsets   [B, n_v, m + 1]    int32: list c of version u is
 *                 out_members[b, u-1, offsets[c] .. offsets[c+1]-1]
 *   out_members   [B, n_v, n_k]      int32 (the first window-size entries used)
 *   out_counts    [B, n_v, n_tiles + 1, m] int32: members of list c below key
 *                 128 t (row n_tiles: the list sizes)
 *   out_assign    optional [B, n_v, n_k] int32: the list of every key of the
 *                 window, -1 beyond it.
 * IDX_EINVAL for n_clusters outside [1, 1024], refit < n_clusters or not a
 * multiple of 128, iters outside [0, 64], or a null required output when
 * n_v >= 1.  With n_k < R (n_v = 0) the outputs are empty, any pointer may
 * be null and nothing is enqueued.  ws: idx_workspace_bytes(p, IDX_OP_IVF_BUILD,
 * 0, n_clusters, 0).
 *
 * idx_ivf_route: group g (as in idx_group_proxy_scan, last member at
 * position p_g) uses version u = floor((p_g + 1) / R).  Its routable keys end
 * at e = u R + b floor((p_g + 1 - u R) / b) (b = insert_batch: keys join
 * their lists in whole batches counted from the refit; e = 0 when u = 0);
 * the keys [e, p_g] are candidates outright.  Clusters are ranked by
 * sum_h wbar[h] * max(0, qbar[h,:] . centroid) with the stored proxy,
 * descending, ties to the lower cluster, and taken in that order with their
 * members below e while those fit in the n_cand - (p_g + 1 - e) slots left;
 * the first cluster that does not fit ends the walk.
 *   centroids/offsets/members/counts: the index idx_ivf_build wrote for the
 *                 same keys, n_clusters and refit (unused when n_k < R).
 *   out_cand      [B, n_g, n_cand] int32: the taken members (cluster by
 *                 cluster), then the keys [e, p_g], then -1.
 *   out_cluster_scores optional [B, n_g, m] float32, -inf without a version.
 *   out_proxy_q/_w     optional, as in idx_group_proxy_scan.
 * IDX_EINVAL also for insert_batch not a positive multiple of 128 or above
 * refit, and n_cand < refit.  ws: idx_workspace_bytes(p, IDX_OP_IVF_ROUTE,
 * group, n_clusters, 0). */
int32_t idx_ivf_build(const idx_problem* p, int32_t n_clusters, int32_t refit, int32_t iters,
                      void* out_centroids, int32_t* out_offsets, int32_t* out_members,
                      int32_t* out_counts, int32_t* out_assign, void* ws, size_t ws_bytes,
                      void* stream);
int32_t idx_ivf_route(const idx_problem* p, int32_t group, int32_t n_clusters, int32_t refit,
                      int32_t insert_batch, int32_t n_cand, const void* centroids,
                      const int32_t* offsets, const int32_t* members, const int32_t* counts,
                      int32_t* out_cand, float* out_cluster_scores, void* out_proxy_q,
                      float* out_proxy_w, void* ws, size_t ws_bytes, void* stream);

/* Kernel timing (measurement aid, off by default).  While enabled, every
 * kernel the library enqueues is bracketed by a pair of HIP events recorded
 * on the same stream; idx_profile_read synchronizes on the recorded events
 * and reports, per kernel kind, the summed duration in milliseconds and the
 * number of launches since the last read (then clears the records).
 * Kinds: 0 dense score scan (the MFMA scan of idx_score_topk, tiled or
 * split-key), 1 select (top-k), 2 proxy build (and block means), 3 reuse
 * (and block expansion), 4 fill (debug score dumps, counter clears), 5 IVF
 * index build (the whole build), 6 IVF routing (cluster scores and list
 * expansion), 7 rescan of the dense scan's overflowed candidate lists,
 * 8 proxy scan (group proxies or block means against the keys), 9 gather
 * scan (PIVOT-Refine re-score of the candidates).  Returns IDX_EHIP on an
 * event error.  Not reentrant: enable it from one host thread only. */
enum { IDX_KERNEL_SCORE = 0, IDX_KERNEL_SELECT = 1, IDX_KERNEL_PROXY = 2, IDX_KERNEL_REUSE = 3,
       IDX_KERNEL_FILL = 4, IDX_KERNEL_IVF_BUILD = 5, IDX_KERNEL_IVF_ROUTE = 6, IDX_KERNEL_RESCAN = 7,
       IDX_KERNEL_PROXY_SCAN = 8, IDX_KERNEL_GATHER_SCAN = 9, IDX_KERNEL_KINDS = 10 };
int32_t idx_profile_enable(int32_t on);
int32_t idx_profile_read(float* ms /* [IDX_KERNEL_KINDS] */, int32_t* launches /* [IDX_KERNEL_KINDS] */);

#ifdef __cplusplus
}
#endif

#endif /* SATC_IDX_H */
