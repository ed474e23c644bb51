// Kernel argument blocks and host-side launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace idx {

constexpr int kSelectThreads = 512;  // 8 waves per select workgroup
constexpr int kSelectCache = 32768;  // row keys kept in LDS by the select (128 KiB)

// Score-kernel modes.
constexpr int kModeDense = 0;   // rows = queries, columns = key positions, row limit q_pos0 + t
constexpr int kModeProxy = 1;   // rows = group proxies, row limit = last member's position
constexpr int kModeGather = 2;  // rows = queries, columns = the group's candidate list
constexpr int kModeList = 3;    // select only: rows are candidate lists (score, key index)
constexpr int kModeBlock = 4;   // rows = group proxies, columns = key blocks (block means)

// Last visible column of row r (-1: none).  Dense: the query's position;
// proxy: the position of the group's last member; block: the last key block
// lying wholly inside that member's prefix (blocks of `block` keys).
__host__ __device__ inline int mode_limit(int mode, int q_pos0, int n_q, int group, int block, int r) {
  if (mode == kModeProxy || mode == kModeBlock) {
    const int last = q_pos0 + ((r + 1) * group < n_q ? (r + 1) * group : n_q) - 1;
    return mode == kModeProxy ? last : (last + 1) / block - 1;
  }
  return q_pos0 + r;
}

// Per-row record a filtering scan leaves for the select: the number of
// candidates, the histogram base (bin = clamp((order key >> 15) - base, 0,
// 2047)), the boundary bin - the highest bin with at least topk candidates
// at or above it (-2: fewer than topk candidates in all; -1: the boundary
// bin holds more than kFiltBoundaryMax of them, or the list was rebuilt by
// a rescan: the select's general path) - and the number of candidates in
// bins above it.  A list holds at most `cld` entries; a row with more
// candidates is pending (status 1) and its exact boundary interval is
// narrowed by rescans: order keys above `hi` (there are exactly `A` of them,
// A < topk) all win, the topk-th largest key lies in [lo, hi].
constexpr int kFiltBins = 2048;  // filter histogram: 256 bins per octave of the score, 8 octaves
constexpr int kFiltInfoCount = 0, kFiltInfoBase = 1, kFiltInfoBoundary = 2, kFiltInfoAbove = 3;
constexpr int kFiltInfoStatus = 4, kFiltInfoLo = 5, kFiltInfoHi = 6, kFiltInfoA = 7;
constexpr int kFiltInfoStride = 8;
constexpr int kFiltBoundaryMax = 256;
// Rescan levels that always resolve a pending row: 11-bit digits of the
// order key (shifts 21, 10, 0), then one pass that keeps the lowest key
// indices of an exactly tied class.
constexpr int kRescanLevels = 4;
// Workgroups of one rescan launch (they loop over the overflowed row blocks).
constexpr int kRescanGrid = 256;

struct ScoreArgs {
  const void* q;          // [B, n_rows, H, D] rows (queries or proxies)
  const float* q_scale;   // [B, n_rows] (FP8 q only)
  const void* k;          // [B, n_k, D]
  const float* k_scale;   // [B, n_k] (FP8 k only)
  const float* w;         // [B, n_rows, H]
  int n_rows, n_k, n_q, q_pos0, group;
  int block;              // key-block size (kModeBlock)
  int n_cols;             // n_k (dense, proxy) or n_cand (gather)
  // [B, n_g, n_cand] (gather only).  A gather workgroup first copies the key
  // indices of its columns [c, c + kc) into LDS (kc <= kCandLdsMax).
  const int* cand;
  int mode;
  int blk0, n_blocks;     // block ids [blk0, blk0 + n_blocks) in this launch
  long long row0;         // flattened row (b * n_rows + r) stored at out row 0
  float* out;             // scores, row stride ld
  long long ld;
  int kc;                 // key columns per workgroup (grid.y = ceil(n_cols / kc))
  int rw;                 // row-waves per workgroup (2, 4, 8); 64 (query, head) rows each
  int nw;                 // waves per workgroup: 8, or 4 (with rw = 4)
  // Candidate filtering (dense scans with one query per wave, whole rows per
  // workgroup): instead of full score rows, each row's candidates - every key
  // whose score reaches the row's running threshold bin - are written as
  // (score, key) pairs at cval/cidx + (row - row0) * cld (at most cld of
  // them), and at ccount + kFiltInfoStride (row - row0) the row's record for
  // the select (see kFiltInfo*): `topk` sets the threshold.  filter = 1: the
  // scan; a workgroup with a row of more than cld candidates appends its
  // block id to ovf_list (ovf_count entries, zero before the scan).
  // filter = 2: the rescan of those blocks (grid.x workgroups loop over the
  // list; rows pending in their records are rescanned, the others skipped).
  int filter;
  float* cval;
  int* cidx;
  int* ccount;
  long long cld;
  int topk;
  int* ovf_count;
  int* ovf_list;
};

struct SelectArgs {
  const float* scores;    // launch row i (flattened row row0 + i) at scores + i * ld
  long long ld;
  long long row0;
  int n_rows;             // rows per sequence (queries or proxies)
  int n_cols;
  int mode;               // kModeDense / kModeProxy: length = limit + 1; kModeGather: all n_cols, -inf = excluded;
                          // kModeList: length = counts[i], key index = lidx[i * ld + c]
  int q_pos0, n_q, group, block;
  const int* cand;        // gather: key index of each column
  const int* lidx;        // list: key indices, same layout as scores
  const int* counts;      // list: entries per launch row
  // filtered lists (when finfo is set; counts is then unused): launch row i's
  // record finfo[kFiltInfoStride i + kFiltInfo*] from the filtering scan
  const int* finfo;
  // segmented list (when seg_counts is set; counts is then unused): launch
  // row i holds seg_counts[i * n_segs + s] entries of segment s at
  // scores/lidx + i * ld + s * seg_len; they are gathered into gval/gidx
  // (same row layout) before the select
  const int* seg_counts;
  int n_segs, seg_len;
  float* gval;
  int* gidx;
  int topk;
  int* out;               // [B * n_rows, topk], indexed by flattened row
};

// Candidate columns one gather workgroup takes (their key indices are staged in LDS).
constexpr int kCandLdsMax = 16384;
constexpr size_t kScoreLdsMax = 160 * 1024;  // LDS of one score workgroup (the CU's whole LDS)
size_t score_lds_bytes(int qf, int kf, int D, int rw, int nw, int filter, int gather_cols);
hipError_t launch_score(const ScoreArgs& a, int qf, int kf, int H, int D, int n_col_chunks,
                        hipStream_t st);
hipError_t launch_select(const SelectArgs& a, int n_launch_rows, hipStream_t st);
// Split-key scan (few rows per sequence, long key axis): see split.hip.
constexpr int kSplitBins = 4096;   // per-row histogram of the top 12 order-key bits
constexpr int kSplitShift = 32 - 12;  // histogram bin = order key >> kSplitShift
constexpr int kSplitWin = 128;     // histogram bins a scan workgroup reports per row
constexpr int kSplitMaxRows = 4;   // rows (queries or proxies) per sequence
constexpr int kMaxSegs = 256;      // segments of a segmented list

// Key-ring geometry of the split-key scan (shared by the kernel and the host
// launcher, which sizes the LDS from it).  A step is 32 key columns; its
// rows are fetched as 1 KiB direct-to-LDS copies, `rwn` row-waves sharing
// them; the ring holds `split_ring_steps` steps per column group.
constexpr int split_step_bytes(int key_bytes, int d) { return 32 * d * key_bytes; }
constexpr int split_dma_waves(int key_bytes, int d, int rwn) {
  return split_step_bytes(key_bytes, d) / 1024 < rwn ? split_step_bytes(key_bytes, d) / 1024 : rwn;
}
// VMEM operations one issuing wave has in flight per step: its share of the
// key copies, plus the key-scale copy of FP8 keys
constexpr int split_ops(int key_bytes, int d, int rwn) {
  return split_step_bytes(key_bytes, d) / 1024 / split_dma_waves(key_bytes, d, rwn) + (key_bytes == 1 ? 1 : 0);
}
constexpr int split_ring_steps(int key_bytes, int d, int rwn) {
  // about 40 KiB of ring (two workgroups fit a CU), at least 4 steps, or 3
  // where 4 would take more than 64 KiB (bf16 keys of d = 128 with one
  // row-wave: four column groups; the histograms of four rows need the rest)
  const int by_lds0 = (40 * 1024) / ((4 / rwn) * split_step_bytes(key_bytes, d));
  const int min_steps = (4 / rwn) * split_step_bytes(key_bytes, d) * 4 <= 64 * 1024 ? 4 : 3;
  const int by_lds = by_lds0 < min_steps ? min_steps : by_lds0;
  const int by_cnt = 2 + 63 / split_ops(key_bytes, d, rwn);                       // vmcnt holds 63
  const int p = by_lds < by_cnt ? by_lds : by_cnt;
  return p > 16 ? 16 : p;
}
// LDS bytes of a split-scan workgroup: ring, per-wave key-scale rings (FP8
// keys), chunk scores, 16-bit-packed histograms, each row's top counted bin
// (within a final 1 KiB).
constexpr size_t split_lds_bytes(int key_bytes, int d, int rwn, int n_rows, int kc) {
  return (size_t)(4 / rwn) * split_ring_steps(key_bytes, d, rwn) * split_step_bytes(key_bytes, d) +
         (key_bytes == 1 ? (size_t)4 * split_ring_steps(key_bytes, d, rwn) * 256 : 0) +
         (size_t)n_rows * kc * 4 + (size_t)n_rows * (kSplitBins / 2) * 4 + 4 * 2 * 32 * 4;
}
constexpr size_t kSplitLdsMax = 160 * 1024;

struct SplitArgs {
  const void* q;          // [B, n_rows, H, D]
  const float* q_scale;   // [B, n_rows] (FP8 q only)
  const void* k;          // [B, n_k, D]
  const float* k_scale;   // [B, n_k] (FP8 k only)
  const float* w;         // [B, n_rows, H]
  int n_rows, n_k, n_q, q_pos0, group, mode;  // mode: kModeDense, kModeProxy or kModeBlock
  int block;              // key-block size (kModeBlock)
  int rwn;                // 64-row waves per workgroup for the rows (1, 2 or 4)
  int kc;                 // key columns per workgroup (grid.x = ceil(n_k / kc)), a multiple of 32 * (4 / rwn)
  float* out;             // [B * n_rows, n_k] scores (-inf: masked)
  // per (row, chunk): the chunk's histogram bins [wbase, wbase + kSplitWin)
  // of that row, wbase = max(top non-empty bin - kSplitWin + 1, 0), or -1
  // when the chunk holds no eligible score of the row
  uint32_t* win;          // [B * n_rows, n_chunks, kSplitWin]
  int* wbase;             // [B * n_rows, n_chunks]
  int n_chunks;
};

struct CompactArgs {
  const float* scores;    // [B * n_rows, n_k]
  const uint32_t* win;    // as SplitArgs
  const int* wbase;
  int n_chunks;
  int n_rows, n_k, n_q, q_pos0, group, mode, topk;
  int block;              // key-block size (kModeBlock)
  int seg;                // columns per workgroup (grid.x = n_segs = ceil(n_k / seg))
  int n_segs;
  float* cval;            // [B * n_rows, n_k]: segment s's candidates from s * seg
  int* cidx;              // [B * n_rows, n_k] their key indices
  int* segcnt;            // [B * n_rows, n_segs] candidates per segment
  int* thr;               // [B * n_rows] each row's threshold bin (order key >> kSplitShift)
};

hipError_t launch_split_scan(const SplitArgs& a, int qf, int kf, int H, int D, int B, int chunks,
                             hipStream_t st);
hipError_t launch_split_compact(const CompactArgs& a, int rows, hipStream_t st);
// Top-k of the split-key scan's rows from the compaction's candidate lists
// and threshold bins (see select.hip): `a` describes the rows (mode,
// positions, n_rows, n_cols = n_k, topk, out) and the segmented lists
// (scores/lidx, seg_counts, n_segs, seg_len, ld = n_k, gval/gidx scratch).
hipError_t launch_split_select(const SelectArgs& a, const int* thr, int rows, hipStream_t st);
hipError_t launch_fill(float* p, size_t n, float v, hipStream_t st);
hipError_t launch_proxy_build(const void* q, const float* q_scale, const float* w, int B, int n_q,
                              int H, int D, int qf, int group, void* pq, float* pw,
                              hipStream_t st);
hipError_t launch_reuse(const int* ptop, int B, int n_q, int q_pos0, int group, int topk,
                        int* out, hipStream_t st);
hipError_t launch_block_means(const void* k, const float* k_scale, int B, int n_k, int D, int kf,
                              int block, void* kbar, hipStream_t st);
hipError_t launch_block_expand(const int* sel, int B, int n_q, int q_pos0, int group, int block,
                               int n_sel, int* cand, hipStream_t st);

// IVF routing (see ivf.hip).
constexpr int kIvfTile = 128;          // keys per assignment workgroup; granularity of the prefix counts
constexpr int kIvfMaxClusters = 1024;  // clusters per version

// One assignment pass over keys [0, n_assign) of every sequence: nearest
// centroid, then the stable inverted lists.  *_bs: per-sequence strides in
// elements.
struct IvfPassArgs {
  const void* k;          // [B, n_k, D]
  const float* k_scale;   // [B, n_k] (FP8 keys only)
  int n_k, m, n_assign;
  const void* cent;       // [m, D] stored centroids (bfloat16, float32 for float32 keys)
  long long cent_bs;
  int* assign;            // [n_assign] nearest centroid
  long long assign_bs;
  int* rank;              // [n_assign] rank among the same-cluster keys of its 128-key tile
  long long rank_bs;
  int* tilecnt;           // [n_tiles, m] keys per (tile, cluster)
  long long tilecnt_bs;
  int* counts;            // [n_tiles + 1, m] members in tiles before t; row n_tiles = list sizes
  long long counts_bs;
  int* offsets;           // [m + 1] list starts
  long long offsets_bs;
  int* members;           // [n_assign] keys grouped by cluster, ascending within a list
  long long members_bs;
};

struct IvfUpdateArgs {
  const void* k;
  const float* k_scale;
  int n_k, m;
  int copy_only;          // 1: dst = src for every cluster
  const int* offsets;     // lists of the assignment to src
  long long offsets_bs;
  const int* members;
  long long members_bs;
  const void* src;        // [m, D] stored centroids before the update
  long long src_bs;
  void* dst;              // [m, D] after (may equal src)
  long long dst_bs;
};

struct IvfRouteArgs {
  const void* pq;         // [B, n_g, H, D] stored proxies
  const float* pw;        // [B, n_g, H]
  const void* cents;      // index: [B, n_v, m, D]
  const int* offsets;     // index: [B, n_v, m + 1]
  const int* members;     // index: [B, n_v, n_k]
  const int* counts;      // index: [B, n_v, n_tiles + 1, m]
  int n_v, m, n_k, n_tiles, n_g, n_q, q_pos0, group, refit, batch, n_cand;
  float* scores;          // [B, n_g, m] cluster scores (-inf without a version)
  int* cand;              // [B, n_g, n_cand]
};

hipError_t launch_fill_i32(int* p, size_t n, int v, hipStream_t st);

// The fixed device scratch of the no-allocation entry point (see
// static_scratch.hip): its size, and its address on the current device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch_ptr(void** out);
hipError_t launch_ivf_init(const void* k, const float* k_scale, int kf, int B, int n_k, int D, int m, int R,
                           void* dst, long long dst_bs, hipStream_t st);
hipError_t launch_ivf_pass(const IvfPassArgs& a, int kf, int D, int B, hipStream_t st);
hipError_t launch_ivf_update(const IvfUpdateArgs& a, int kf, int D, int B, hipStream_t st);
hipError_t launch_ivf_route(const IvfRouteArgs& a, int cf, int H, int D, int B, hipStream_t st);

}  // namespace idx
