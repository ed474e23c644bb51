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

struct ScoreArgs {
  const void* q;          // [B, n_rows, H, D] rows (queries or proxies)
  const float* q_scale;   // [B, n_rows] (FP8 q only)
  const void* k;          // [B, n_k, D]
  const float* k_scale;   // [B, n_k] (FP8 k only)
  const float* w;         // [B, n_rows, H]
  int n_rows, n_k, n_q, q_pos0, group;
  int n_cols;             // n_k (dense, proxy) or n_cand (gather)
  const int* cand;        // [B, n_g, n_cand] (gather only)
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
  // (score, key) pairs at cval/cidx + (row - row0) * cld and their number at
  // ccount[row - row0].  `topk` sets the threshold.
  int filter;
  float* cval;
  int* cidx;
  int* ccount;
  long long cld;
  int topk;
};

struct SelectArgs {
  const float* scores;    // launch row i (flattened row row0 + i) at scores + i * ld
  long long ld;
  long long row0;
  int n_rows;             // rows per sequence (queries or proxies)
  int n_cols;
  int mode;               // kModeDense / kModeProxy: length = limit + 1; kModeGather: all n_cols, -inf = excluded;
                          // kModeList: length = counts[i], key index = lidx[i * ld + c]
  int q_pos0, n_q, group;
  const int* cand;        // gather: key index of each column
  const int* lidx;        // list: key indices, same layout as scores
  const int* counts;      // list: entries per launch row
  int topk;
  int* out;               // [B * n_rows, topk], indexed by flattened row
};

size_t score_lds_bytes(int qf, int kf, int D, int rw, int nw, int filter);
hipError_t launch_score(const ScoreArgs& a, int qf, int kf, int H, int D, int n_col_chunks,
                        hipStream_t st);
hipError_t launch_select(const SelectArgs& a, int n_launch_rows, hipStream_t st);
hipError_t launch_fill(float* p, size_t n, float v, hipStream_t st);
hipError_t launch_proxy_build(const void* q, const float* q_scale, const float* w, int B, int n_q,
                              int H, int D, int qf, int group, void* pq, float* pw,
                              hipStream_t st);
hipError_t launch_reuse(const int* ptop, int B, int n_q, int q_pos0, int group, int topk,
                        int* out, hipStream_t st);

}  // namespace idx
