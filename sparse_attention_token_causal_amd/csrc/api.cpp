// C ABI of the indexer library: argument checks, workspace carving, kernel
// dispatch.  Every check happens on the host before anything is enqueued.
#include "idx.h"

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "kernels.hpp"

namespace {

using namespace idx;

// ---- optional per-kernel timing with HIP events (measurement aid) ----
struct TimedLaunch {
  int kind;
  hipEvent_t start, stop;
};
bool g_profile = false;
std::vector<TimedLaunch> g_records;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (a callable returning hipError_t), bracketed by events when
// profiling is on.
template <class F>
hipError_t timed(int kind, hipStream_t st, F launch) {
  if (!g_profile) return launch();
  TimedLaunch r{kind, take_event(), take_event()};
  if (!r.start || !r.stop) return hipErrorOutOfMemory;
  (void)hipEventRecord(r.start, st);
  hipError_t e = launch();
  (void)hipEventRecord(r.stop, st);
  g_records.push_back(r);
  return e;
}

constexpr size_t kAlign = 256;
constexpr size_t kScoreBufferTarget = size_t(2) << 30;  // score rows buffered per chunk (bytes)
// Candidate lists of a filtering dense scan buffered per chunk (bytes): the
// workspace of idx_score_topk stays below this (plus a few bytes per row
// block) at any sequence length.
constexpr size_t kListBufferTarget = size_t(4) << 30;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

bool dtype_ok(int d) { return d == IDX_F32 || d == IDX_BF16 || d == IDX_FP8_E4M3; }

bool combo_supported(int qf, int kf, int H, int D) {
  if (!(H == 16 || H == 32 || H == 64)) return false;
  if (!(D == 64 || D == 128)) return false;
  return (qf == IDX_F32 && kf == IDX_F32) || (qf == IDX_BF16 && kf == IDX_BF16) ||
         (qf == IDX_BF16 && kf == IDX_FP8_E4M3) || (qf == IDX_FP8_E4M3 && kf == IDX_FP8_E4M3);
}

// Shape and pointer checks shared by the scoring entry points.
int check_problem(const idx_problem* p) {
  if (!p) return IDX_EINVAL;
  if (p->batch < 1 || p->n_q < 1 || p->n_k < 1 || p->heads < 1 || p->dim < 1) return IDX_EINVAL;
  if (p->q_pos0 < 0 || (long long)p->q_pos0 + p->n_q > p->n_k) return IDX_EINVAL;
  if (!dtype_ok(p->q_dtype) || !dtype_ok(p->k_dtype)) return IDX_EINVAL;
  if (!p->q || !p->k || !p->w) return IDX_EINVAL;
  if ((p->q_dtype == IDX_FP8_E4M3) != (p->q_scale != nullptr)) return IDX_EINVAL;
  if ((p->k_dtype == IDX_FP8_E4M3) != (p->k_scale != nullptr)) return IDX_EINVAL;
  if (!combo_supported(p->q_dtype, p->k_dtype, p->heads, p->dim)) return IDX_EUNSUPPORTED;
  return IDX_OK;
}

// Row-waves per score workgroup: enough 64-row waves for the rows of one
// segment (a sequence or a group), a power of two in [2, 8].
int pick_rw(long long rows_per_segment, int H) {
  const long long waves = (rows_per_segment * H + 63) / 64;
  int rw = 2;
  while (rw < 8 && rw < waves) rw *= 2;
  return rw;
}

int queries_per_block(int rw, int H) { return rw * (64 / H); }

// First flattened row covered by score block `blk` (blk == total -> end).
long long block_start_row(int mode, int blk, int total, int B, int n_rows, int n_q, int group,
                          int BQ) {
  if (blk >= total) return (long long)B * (mode == kModeGather ? n_q : n_rows);
  if (mode != kModeGather) {
    const int bps = ceil_div(n_rows, BQ);
    const int b = blk / bps, r = (blk % bps) * BQ;
    return (long long)b * n_rows + r;
  }
  const int n_g = ceil_div(n_q, group), bpg = ceil_div(group, BQ);
  const int b = blk / (n_g * bpg), g = (blk / bpg) % n_g, j = blk % bpg;
  const int gs = g * group, ge = (gs + group < n_q) ? gs + group : n_q;
  int r = gs + j * BQ;
  if (r > ge) r = ge;
  return (long long)b * n_q + r;
}

struct Layout {
  int mode, rw, nw, BQ, total_blocks, n_rows, n_cols;
  bool filter;  // dense scan with candidate filtering (see ScoreArgs::filter)
};

// The proxies' storage format (and so the proxy scan's q format).
int proxy_q_dtype(const idx_problem* p) { return p->q_dtype == IDX_F32 ? IDX_F32 : IDX_BF16; }

Layout make_layout(int mode, const idx_problem* p, int n_rows, int n_cols, int group) {
  Layout L;
  L.mode = mode;
  L.n_rows = n_rows;
  L.n_cols = n_cols;
  // float32 key tiles of d = 128 fit the LDS only up to 128 columns
  // (two buffers of 256 would take 264 KiB): at least four row-waves then
  const int scan_qf = mode == kModeProxy ? proxy_q_dtype(p) : p->q_dtype;
  const int min_rw = (scan_qf == IDX_F32 && p->dim == 128) ? 4 : 2;
  if (mode == kModeGather) {
    const int seg = group < p->n_q ? group : p->n_q;
    L.rw = std::max(pick_rw(seg, p->heads), min_rw);
    L.BQ = queries_per_block(L.rw, p->heads);
    L.total_blocks = p->batch * ceil_div(p->n_q, group) * ceil_div(group, L.BQ);
  } else {
    L.rw = std::max(pick_rw(n_rows, p->heads), min_rw);
    L.nw = 8;
    L.filter = false;
    // Long dense scans with 64 heads (eight query-waves per workgroup, one
    // query per wave) filter candidates
    if (mode == kModeDense && p->heads == 64 && L.rw == 8) L.filter = true;
    L.BQ = queries_per_block(L.rw, p->heads);
    L.total_blocks = p->batch * ceil_div(n_rows, L.BQ);
    return L;
  }
  L.nw = 8;
  L.filter = false;
  return L;
}

// Rows of the score buffer the workspace should hold for this layout.
long long buffer_rows(const Layout& L, long long total_rows) {
  long long rows = (long long)(kScoreBufferTarget / ((size_t)L.n_cols * 4));
  if (rows < L.BQ) rows = L.BQ;
  const long long padded = (long long)L.total_blocks * L.BQ;
  if (rows > padded) rows = padded;
  if (rows > total_rows + L.BQ) rows = total_rows + L.BQ;
  return (rows + L.BQ - 1) / L.BQ * L.BQ;
}

// Score the rows block-chunk by block-chunk into `buf` and select each row's
// top-k into `out`.  `full` = buf holds every row (row stride n_cols).
// Candidate filtering (see ScoreArgs::filter) replaces full score rows by
// per-row candidate lists in dense scans with one query per wave.
struct Filter {
  bool on = false;
  int cap = 0;              // list capacity (entries per row)
  float* val = nullptr;     // [rows, cap]
  int* idx = nullptr;       // [rows, cap]
  int* count = nullptr;     // [rows, kFiltInfoStride] records
  int* ovf_cnt = nullptr;   // one overflow counter per chunk
  int* ovf_list = nullptr;  // [blocks per chunk] overflowed row blocks of the current chunk
};

// grec (gathered columns only, may be null): [buf_rows, kFiltInfoStride]
// records of each row's exact boundary bin, written by the scan when one
// workgroup sees a row's every column, for the select's one-pass path.
int score_and_select(ScoreArgs sa, const Layout& L, int qf, int kf, int H, int D, int B, int n_q,
                     int group, float* buf, long long buf_rows, bool full, int topk, int* out,
                     hipStream_t st, const Filter& flt = Filter(), int* grec = nullptr) {
  const int bpc_max = full ? L.total_blocks : (int)(buf_rows / L.BQ);
  if (bpc_max < 1) return IDX_EWORKSPACE;
  // chunks of equal size (a short last chunk would run a launch of a few
  // workgroups of the longest rows)
  const int bpc = ceil_div(L.total_blocks, ceil_div(L.total_blocks, bpc_max));
  const int tw = (L.nw / L.rw) * 64;
  if (flt.on) {
    // the overflow counters of every chunk start at zero (a fill kernel: no
    // memset, so that the call can be captured in a graph)
    const int n_chunks = ceil_div(L.total_blocks, bpc);
    if (timed(IDX_KERNEL_FILL, st, [&] { return launch_fill_i32(flt.ovf_cnt, (size_t)n_chunks, 0, st); }) !=
        hipSuccess)
      return IDX_EHIP;
  }
  for (int blk0 = 0; blk0 < L.total_blocks; blk0 += bpc) {
    const int nb = (L.total_blocks - blk0 < bpc) ? L.total_blocks - blk0 : bpc;
    const long long r0 = block_start_row(L.mode, blk0, L.total_blocks, B, L.n_rows, n_q, group, L.BQ);
    const long long r1 = block_start_row(L.mode, blk0 + nb, L.total_blocks, B, L.n_rows, n_q, group, L.BQ);
    if (r1 <= r0) continue;
    // Split the key columns when there are few row blocks: aim for about
    // eight workgroups per CU with at least 16 key tiles each (the causal
    // limit leaves the chunks beyond a row block's last key empty, so the
    // busy ones number far fewer: the proxy scans of long sequences, whose
    // 2048 proxies make 256 row blocks), and for at least one per CU on short
    // scans.  Filtering keeps whole rows in one workgroup.
    int chunks = 1;
    if (nb < 2048 && !flt.on) {
      chunks = std::max(1, std::min(ceil_div(2048, nb), ceil_div(L.n_cols, 16 * tw)));
      if ((long long)nb * chunks < 256) chunks = std::min(ceil_div(256, nb), ceil_div(L.n_cols, tw));
    }
    int kc = ceil_div(L.n_cols, chunks);
    kc = ceil_div(kc, tw) * tw;
    // a gather workgroup stages its columns' key indices in LDS, beside the
    // key tiles
    if (L.mode == kModeGather) {
      const size_t tiles = score_lds_bytes(qf, kf, D, L.rw, L.nw, 0, 0);
      const int fit = (int)((kScoreLdsMax - tiles) / 4) / tw * tw;
      kc = std::min(kc, std::min(kCandLdsMax, fit));
    }
    chunks = ceil_div(L.n_cols, kc);
    const bool recs = grec && L.mode == kModeGather && chunks == 1 && H == 64 && L.rw == 8 &&
                      score_lds_bytes(qf, kf, D, L.rw, L.nw, 3, kc) <= kScoreLdsMax;
    sa.blk0 = blk0;
    sa.n_blocks = nb;
    sa.row0 = full ? 0 : r0;
    sa.out = buf;
    sa.ld = L.n_cols;
    sa.kc = kc;
    sa.rw = L.rw;
    sa.nw = L.nw;
    sa.filter = flt.on ? 1 : (recs ? 3 : 0);
    sa.cval = flt.val;
    sa.cidx = flt.idx;
    sa.ccount = recs ? grec : flt.count;
    sa.cld = flt.on ? flt.cap : L.n_cols;
    sa.topk = topk;
    sa.ovf_count = flt.on ? flt.ovf_cnt + blk0 / bpc : nullptr;
    sa.ovf_list = flt.ovf_list;
    const int kind = L.mode == kModeGather ? IDX_KERNEL_GATHER_SCAN
                     : (L.mode == kModeDense ? IDX_KERNEL_SCORE : IDX_KERNEL_PROXY_SCAN);
    if (timed(kind, st, [&] { return launch_score(sa, qf, kf, H, D, chunks, st); }) != hipSuccess)
      return IDX_EHIP;
    if (flt.on) {
      // rows whose candidates overflowed their list: a fixed grid of
      // workgroups rescans the listed row blocks (none: it exits at once)
      ScoreArgs rs = sa;
      rs.filter = 2;
      rs.n_blocks = std::min(nb, kRescanGrid);
      if (timed(IDX_KERNEL_RESCAN, st, [&] { return launch_score(rs, qf, kf, H, D, 1, st); }) != hipSuccess)
        return IDX_EHIP;
    }
    SelectArgs se = {};
    se.scores = buf + (full ? r0 * (long long)L.n_cols : 0);
    se.ld = L.n_cols;
    se.row0 = r0;
    se.n_rows = (L.mode == kModeGather) ? n_q : L.n_rows;
    se.n_cols = L.n_cols;
    se.mode = L.mode;
    se.q_pos0 = sa.q_pos0;
    se.n_q = n_q;
    se.group = group;
    se.block = sa.block;
    se.cand = sa.cand;
    se.lidx = nullptr;
    se.counts = nullptr;
    se.finfo = recs ? grec : nullptr;
    se.topk = topk;
    se.out = out;
    if (flt.on) {
      se.mode = kModeList;
      se.scores = flt.val;
      se.lidx = flt.idx;
      se.finfo = flt.count;
      se.ld = flt.cap;
      se.n_cols = flt.cap;
    }
    if (timed(IDX_KERNEL_SELECT, st, [&] { return launch_select(se, (int)(r1 - r0), st); }) != hipSuccess)
      return IDX_EHIP;
  }
  return IDX_OK;
}

ScoreArgs base_args(const idx_problem* p) {
  ScoreArgs a = {};
  a.q = p->q;
  a.q_scale = p->q_scale;
  a.k = p->k;
  a.k_scale = p->k_scale;
  a.w = p->w;
  a.n_rows = p->n_q;
  a.n_k = p->n_k;
  a.n_q = p->n_q;
  a.q_pos0 = p->q_pos0;
  a.group = 1;
  a.block = 1;
  a.n_cols = p->n_k;
  a.cand = nullptr;
  a.mode = kModeDense;
  return a;
}

// Long dense scans with 64 heads (one query per wave) filter candidates
// instead of writing full score rows.
bool use_filter(const idx_problem* p, const Layout& L) { return L.filter && p->heads == 64; }

// Entries a filtered candidate list holds.  A running top-k threshold over n
// keys in random order admits about k (1 + ln(n / k)) of them, and every key
// passes until the threshold first moves (at least topk keys, checked every
// eight 64-key tiles).  On the 32K, 131K and 262K prefill workloads the
// largest row held 8175, 11099 and 12569 candidates, at most 584 above that
// estimate: the capacity is 1.25 times the estimate plus 1024 (28-31% above
// those maxima), at least topk (a rescan cuts a tied class to exactly topk
// entries) and at most n_k.  A row with more candidates is resolved exactly
// by the rescan.
int list_cap(int n_k, int topk) {
  if (topk >= n_k) return n_k;
  const double e = 1.25 * topk * (1.0 + std::log((double)n_k / topk)) + 1024.0;
  long long c = ((long long)std::ceil(e) + 255) / 256 * 256;
  if (c < topk) c = topk;
  return (int)std::min<long long>(c, n_k);
}

// Workspace of a filtering dense scan: the overflow counters (one per chunk)
// and the overflow list (one slot per row block), then for `rows` buffered
// rows their lists ([rows, cap] scores, [rows, cap] keys) and records
// ([rows, kFiltInfoStride] ints).
struct FilterLayout {
  int cap;
  size_t row_bytes, fixed;
  long long target_rows;  // rows the workspace buffers at the library's own size
};

FilterLayout filter_layout(const idx_problem* p, const Layout& L, int topk) {
  FilterLayout F;
  F.cap = list_cap(p->n_k, topk);
  F.row_bytes = (size_t)F.cap * 8 + (size_t)kFiltInfoStride * 4;
  F.fixed = 2 * align_up((size_t)L.total_blocks * 4);
  long long rows = (long long)(kListBufferTarget / F.row_bytes) / L.BQ * L.BQ;
  rows = std::max<long long>(rows, L.BQ);
  rows = std::min<long long>(rows, (long long)L.total_blocks * L.BQ);
  F.target_rows = rows;
  return F;
}

// Carves a filtering scan's workspace; returns the rows it buffers (0: too small).
long long carve_filter(const FilterLayout& F, const Layout& L, char* ws, size_t ws_bytes, Filter& flt) {
  if (ws_bytes < F.fixed + (size_t)L.BQ * F.row_bytes) return 0;
  const long long rows = (long long)((ws_bytes - F.fixed) / F.row_bytes);
  flt.on = true;
  flt.cap = F.cap;
  flt.ovf_cnt = (int*)ws;
  flt.ovf_list = (int*)(ws + F.fixed / 2);
  char* lists = ws + F.fixed;
  flt.val = (float*)lists;
  flt.idx = (int*)(lists + (size_t)rows * F.cap * 4);
  flt.count = (int*)(lists + (size_t)rows * F.cap * 8);
  return rows;
}

size_t proxy_q_bytes(const idx_problem* p, int n_g) {
  return (size_t)p->batch * n_g * p->heads * p->dim * (proxy_q_dtype(p) == IDX_F32 ? 4 : 2);
}


// Short row sets (at most kSplitMaxRows queries or proxies per sequence, the
// decode shape) take the split-key scan with the histogram / compaction /
// list select.  `qf` is the format the scan reads q in.
bool split_shape(const idx_problem* p, int n_rows, int qf) {
  return n_rows <= kSplitMaxRows && qf != IDX_F32 && p->k_dtype != IDX_F32;
}

// 64-row waves the rows of one sequence need in the split-key scan (1, 2 or 4).
int split_rwn(const idx_problem* p, int n_rows) {
  const int waves = ceil_div((long long)n_rows * p->heads, 64);
  return waves <= 1 ? 1 : (waves <= 2 ? 2 : 4);
}

// Key columns per split-scan workgroup: a multiple of the column-group step,
// aiming at one round of two workgroups per CU, else of one, else the
// largest chunk the LDS holds.
int split_kc(const idx_problem* p, int n_rows) {
  const int rwn = split_rwn(p, n_rows), gran = 32 * (4 / rwn);
  const int kb = p->k_dtype == IDX_FP8_E4M3 ? 1 : 2;
  for (int per_cu = 2; per_cu >= 1; --per_cu) {
    const int chunks = std::max(1, std::min(ceil_div(256 * per_cu, p->batch), ceil_div(p->n_k, gran)));
    const int kc = ceil_div(ceil_div(p->n_k, chunks), gran) * gran;
    if (split_lds_bytes(kb, p->dim, rwn, n_rows, kc) * per_cu <= kSplitLdsMax) return kc;
  }
  const size_t fixed = split_lds_bytes(kb, p->dim, rwn, n_rows, 0);
  return std::max(gran, (int)((kSplitLdsMax - fixed) / (4 * (size_t)n_rows)) / gran * gran);
}

// Compaction segments: about 512 workgroups over all rows, at most kMaxSegs per row.
int split_seg(const idx_problem* p, int n_rows) {
  const int R = p->batch * n_rows;
  int seg = std::max(1024, ceil_div(ceil_div(p->n_k, ceil_div(512, R)), 256) * 256);
  if (ceil_div(p->n_k, seg) > kMaxSegs) seg = ceil_div(ceil_div(p->n_k, kMaxSegs), 256) * 256;
  return seg;
}

struct SplitLayout {
  int kc, chunks, seg, segs;
  size_t scores, win, wbase, cval, cidx, segcnt, gval, gidx, thr, total;  // byte offsets
};

// Region, R = B * n_rows: [R, n_k] scores | [R, chunks, kSplitWin] windows |
// [R, chunks] window bases | [R, n_k] candidate scores | [R, n_k] candidate
// keys | [R, segs] segment counts | [R, n_k] gathered scores | [R, n_k]
// gathered keys | [R] threshold bins.
SplitLayout split_layout(const idx_problem* p, int n_rows) {
  const size_t R = (size_t)p->batch * n_rows, row = (size_t)p->n_k * 4;
  SplitLayout s;
  s.kc = split_kc(p, n_rows);
  s.chunks = ceil_div(p->n_k, s.kc);
  s.seg = split_seg(p, n_rows);
  s.segs = ceil_div(p->n_k, s.seg);
  size_t o = 0;
  s.scores = o;  o += align_up(R * row);
  s.win = o;     o += align_up(R * s.chunks * kSplitWin * 4);
  s.wbase = o;   o += align_up(R * s.chunks * 4);
  s.cval = o;    o += align_up(R * row);
  s.cidx = o;    o += align_up(R * row);
  s.segcnt = o;  o += align_up(R * s.segs * 4);
  s.gval = o;    o += align_up(R * row);
  s.gidx = o;    o += align_up(R * row);
  s.thr = o;     o += align_up(R * 4);
  s.total = o;
  return s;
}

// Split-key scan of n_rows rows per sequence, then the top-`topk` of each row
// into out [B * n_rows, topk].  `scores` (if non-null) receives the scores
// (already filled with -inf by the caller); otherwise the region's own
// buffer holds them.
int split_score_select(const idx_problem* p, int qf, const void* q, const float* q_scale,
                       const float* w, int n_rows, int mode, int group, int block, int topk,
                       int* out, float* scores, char* region, hipStream_t st) {
  const SplitLayout sl = split_layout(p, n_rows);
  const int B = p->batch, R = B * n_rows;
  if (!scores) scores = (float*)(region + sl.scores);
  SplitArgs a = {};
  a.q = q;
  a.q_scale = q_scale;
  a.k = p->k;
  a.k_scale = p->k_scale;
  a.w = w;
  a.n_rows = n_rows;
  a.n_k = p->n_k;
  a.n_q = p->n_q;
  a.q_pos0 = p->q_pos0;
  a.group = group;
  a.mode = mode;
  a.block = block;
  a.rwn = split_rwn(p, n_rows);
  a.kc = sl.kc;
  a.out = scores;
  a.win = (uint32_t*)(region + sl.win);
  a.wbase = (int*)(region + sl.wbase);
  a.n_chunks = sl.chunks;
  if (timed(mode == kModeDense ? IDX_KERNEL_SCORE : IDX_KERNEL_PROXY_SCAN, st, [&] {
        return launch_split_scan(a, qf, p->k_dtype, p->heads, p->dim, B, sl.chunks, st);
      }) != hipSuccess)
    return IDX_EHIP;
  CompactArgs c = {};
  c.scores = scores;
  c.win = a.win;
  c.wbase = a.wbase;
  c.n_chunks = sl.chunks;
  c.n_rows = n_rows;
  c.n_k = p->n_k;
  c.n_q = p->n_q;
  c.q_pos0 = p->q_pos0;
  c.group = group;
  c.mode = mode;
  c.block = block;
  c.topk = topk;
  c.seg = sl.seg;
  c.n_segs = sl.segs;
  c.cval = (float*)(region + sl.cval);
  c.cidx = (int*)(region + sl.cidx);
  c.segcnt = (int*)(region + sl.segcnt);
  c.thr = (int*)(region + sl.thr);
  SelectArgs se = {};
  se.scores = c.cval;
  se.ld = p->n_k;
  se.row0 = 0;
  se.n_rows = n_rows;
  se.n_cols = p->n_k;
  se.mode = mode;
  se.q_pos0 = p->q_pos0;
  se.n_q = p->n_q;
  se.group = group;
  se.block = block;
  se.lidx = c.cidx;
  se.seg_counts = c.segcnt;
  se.n_segs = sl.segs;
  se.seg_len = sl.seg;
  se.gval = (float*)(region + sl.gval);
  se.gidx = (int*)(region + sl.gidx);
  se.topk = topk;
  se.out = out;
  if (timed(IDX_KERNEL_SELECT, st, [&] {
        hipError_t e = launch_split_compact(c, R, st);
        return e != hipSuccess ? e : launch_split_select(se, c.thr, R, st);
      }) != hipSuccess)
    return IDX_EHIP;
  return IDX_OK;
}


// Block routing: the block-mean "keys" the proxy scans (bfloat16, float32
// for float32 keys) and the problem that scan is: the group proxies against
// n_b = ceil(n_k / block) block means, positions unchanged.
int block_mean_dtype(const idx_problem* p) { return p->k_dtype == IDX_F32 ? IDX_F32 : IDX_BF16; }

idx_problem block_problem(const idx_problem* p, int block, const void* pq, const float* pw,
                          const void* kbar) {
  idx_problem q = *p;
  q.n_k = ceil_div(p->n_k, block);
  q.q_dtype = proxy_q_dtype(p);
  q.k_dtype = block_mean_dtype(p);
  q.q = pq;
  q.q_scale = nullptr;
  q.k = kbar;
  q.k_scale = nullptr;
  q.w = pw;
  return q;
}

struct BlockLayout {
  size_t pq, pw, kbar, sel, scan, total;  // byte offsets
  bool split;
  long long rows;  // score rows the tiled scan's buffer holds
};

BlockLayout block_layout(const idx_problem* p, int group, int block, int n_sel) {
  const int n_g = ceil_div(p->n_q, group);
  const idx_problem q = block_problem(p, block, nullptr, nullptr, nullptr);
  BlockLayout L;
  size_t o = 0;
  L.pq = o;   o += align_up(proxy_q_bytes(p, n_g));
  L.pw = o;   o += align_up((size_t)p->batch * n_g * p->heads * 4);
  L.kbar = o; o += align_up((size_t)p->batch * q.n_k * p->dim * (q.k_dtype == IDX_F32 ? 4 : 2));
  L.sel = o;  o += align_up((size_t)p->batch * n_g * n_sel * 4);
  L.scan = o;
  L.split = split_shape(&q, n_g, q.q_dtype);
  if (L.split) {
    L.rows = 0;
    o += split_layout(&q, n_g).total;
  } else {
    Layout S = make_layout(kModeBlock, &q, n_g, q.n_k, group);
    L.rows = buffer_rows(S, (long long)p->batch * n_g);
    o += align_up((size_t)L.rows * q.n_k * 4);
  }
  L.total = o;
  return L;
}

// IVF routing: centroids are stored like the proxy (float32 for float32
// keys, bfloat16 otherwise); lists and counts are int32.
int ivf_cent_dtype(const idx_problem* p) { return p->k_dtype == IDX_F32 ? IDX_F32 : IDX_BF16; }
size_t ivf_cent_elt(const idx_problem* p) { return ivf_cent_dtype(p) == IDX_F32 ? 4 : 2; }
int ivf_tiles(int n) { return ceil_div(n, kIvfTile); }

// Checks of the key fields an index build reads (q and w are not read).
int check_keys(const idx_problem* p) {
  if (!p) return IDX_EINVAL;
  if (p->batch < 1 || p->n_k < 1 || p->dim < 1 || !dtype_ok(p->k_dtype) || !p->k) return IDX_EINVAL;
  if ((p->k_dtype == IDX_FP8_E4M3) != (p->k_scale != nullptr)) return IDX_EINVAL;
  if (!(p->dim == 64 || p->dim == 128)) return IDX_EUNSUPPORTED;
  return IDX_OK;
}

bool ivf_params_ok(int m, int refit) {
  return m >= 1 && m <= kIvfMaxClusters && refit >= m && refit % kIvfTile == 0;
}

// Build workspace: the initial centroids, per-key cluster and in-tile rank,
// per-tile counts, and the lists of the assignment passes that are not
// published (offsets, members, prefix counts).
struct IvfBuildLayout {
  size_t cur, rank, assign, tilecnt, counts, offsets, members, total;
};

IvfBuildLayout ivf_build_layout(const idx_problem* p, int m) {
  const size_t B = p->batch, n_k = p->n_k, nt = ivf_tiles(p->n_k);
  IvfBuildLayout L;
  size_t o = 0;
  L.cur = o;     o += align_up(B * m * p->dim * ivf_cent_elt(p));
  L.rank = o;    o += align_up(B * n_k * 4);
  L.assign = o;  o += align_up(B * n_k * 4);
  L.tilecnt = o; o += align_up(B * nt * m * 4);
  L.counts = o;  o += align_up(B * (nt + 1) * m * 4);
  L.offsets = o; o += align_up(B * (m + 1) * 4);
  L.members = o; o += align_up(B * n_k * 4);
  L.total = o;
  return L;
}

// Route workspace: the stored proxies and the cluster scores.
struct IvfRouteLayout {
  size_t pq, pw, scores, total;
};

IvfRouteLayout ivf_route_layout(const idx_problem* p, int group, int m) {
  const int n_g = ceil_div(p->n_q, group);
  IvfRouteLayout L;
  size_t o = 0;
  L.pq = o;     o += align_up(proxy_q_bytes(p, n_g));
  L.pw = o;     o += align_up((size_t)p->batch * n_g * p->heads * 4);
  L.scores = o; o += align_up((size_t)p->batch * n_g * m * 4);
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

int32_t idx_version(void) { return 100; }

const char* idx_status_string(int32_t s) {
  switch (s) {
    case IDX_OK: return "ok";
    case IDX_EINVAL: return "invalid argument";
    case IDX_EUNSUPPORTED: return "unsupported heads/dim/dtype combination";
    case IDX_EWORKSPACE: return "workspace too small";
    case IDX_EHIP: return "HIP launch error";
    case IDX_ETOOLARGE: return "problem needs more scratch than the fixed device array of the no-allocation entry point";
    default: return "unknown status";
  }
}

size_t idx_workspace_bytes(const idx_problem* p, int32_t op, int32_t group, int32_t n_cand,
                           int32_t topk) {
  (void)topk;
  if (op == IDX_OP_REUSE_TOPK) return 0;
  if (op == IDX_OP_IVF_BUILD) {  // n_cand = clusters per version; only the key fields are read
    if (check_keys(p) != IDX_OK || n_cand < 1 || n_cand > kIvfMaxClusters) return 0;
    return ivf_build_layout(p, n_cand).total;
  }
  if (check_problem(p) != IDX_OK) return 0;
  if (op == IDX_OP_SCORE_TOPK) {
    if (split_shape(p, p->n_q, p->q_dtype)) return split_layout(p, p->n_q).total;
    Layout L = make_layout(kModeDense, p, p->n_q, p->n_k, 1);
    if (use_filter(p, L)) {
      if (topk < 1) return 0;
      const FilterLayout F = filter_layout(p, L, topk);
      return F.fixed + align_up((size_t)F.target_rows * F.row_bytes);
    }
    return align_up((size_t)buffer_rows(L, (long long)p->batch * p->n_q) * (size_t)p->n_k * 4);
  }
  if (group < 1) return 0;
  const int n_g = ceil_div(p->n_q, group);
  if (op == IDX_OP_GROUP_PROXY_SCAN) {
    const size_t proxy = align_up(proxy_q_bytes(p, n_g)) + align_up((size_t)p->batch * n_g * p->heads * 4);
    if (split_shape(p, n_g, proxy_q_dtype(p))) return proxy + split_layout(p, n_g).total;
    Layout L = make_layout(kModeProxy, p, n_g, p->n_k, group);
    return proxy + align_up((size_t)buffer_rows(L, (long long)p->batch * n_g) * p->n_k * 4);
  }
  if (op == IDX_OP_BLOCK_ROUTE) {  // n_cand = block size, topk = blocks kept
    if (n_cand < 1 || topk < 1) return 0;
    return block_layout(p, group, n_cand, topk).total;
  }
  if (op == IDX_OP_IVF_ROUTE) {  // n_cand = clusters per version
    if (n_cand < 1 || n_cand > kIvfMaxClusters) return 0;
    return ivf_route_layout(p, group, n_cand).total;
  }
  if (op == IDX_OP_REFINE_TOPK) {
    if (n_cand < 1) return 0;
    Layout L = make_layout(kModeGather, p, p->n_q, n_cand, group);
    const long long rows = buffer_rows(L, (long long)p->batch * p->n_q);
    return align_up((size_t)rows * n_cand * 4) + align_up((size_t)rows * kFiltInfoStride * 4);
  }
  return 0;
}

int32_t idx_score_topk(const idx_problem* p, int32_t topk, int32_t* out_idx, float* out_scores,
                       void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != IDX_OK) return rc;
  if (topk < 1 || !out_idx) return IDX_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  const bool full = out_scores != nullptr;
  if (split_shape(p, p->n_q, p->q_dtype)) {
    const size_t need = idx_workspace_bytes(p, IDX_OP_SCORE_TOPK, 0, 0, topk);
    if (!ws || ws_bytes < need) return IDX_EWORKSPACE;
    if (full && timed(IDX_KERNEL_FILL, st, [&] {
          return launch_fill(out_scores, (size_t)p->batch * p->n_q * p->n_k, -__builtin_huge_valf(), st);
        }) != hipSuccess)
      return IDX_EHIP;
    return split_score_select(p, p->q_dtype, p->q, p->q_scale, p->w, p->n_q, kModeDense, 1, 1, topk,
                              out_idx, out_scores, (char*)ws, st);
  }
  Layout L = make_layout(kModeDense, p, p->n_q, p->n_k, 1);
  float* buf;
  long long rows;
  if (full) {
    buf = out_scores;
    rows = (long long)p->batch * p->n_q;
    if (timed(IDX_KERNEL_FILL, st, [&] {
          return launch_fill(out_scores, (size_t)rows * p->n_k, -__builtin_huge_valf(), st);
        }) != hipSuccess)
      return IDX_EHIP;
  }
  ScoreArgs sa = base_args(p);
  if (full)
    return score_and_select(sa, L, p->q_dtype, p->k_dtype, p->heads, p->dim, p->batch, p->n_q, 1,
                            buf, rows, full, topk, out_idx, st);
  const size_t need = idx_workspace_bytes(p, IDX_OP_SCORE_TOPK, 0, 0, topk);
  if (!ws || ws_bytes < need) return IDX_EWORKSPACE;
  if (!use_filter(p, L)) {
    rows = (long long)(ws_bytes / ((size_t)p->n_k * 4));
    return score_and_select(sa, L, p->q_dtype, p->k_dtype, p->heads, p->dim, p->batch, p->n_q, 1,
                            (float*)ws, rows, false, topk, out_idx, st);
  }
  // a larger workspace buffers more rows per chunk (fewer launches)
  Filter flt;
  rows = carve_filter(filter_layout(p, L, topk), L, (char*)ws, ws_bytes, flt);
  if (rows < L.BQ) return IDX_EWORKSPACE;
  return score_and_select(sa, L, p->q_dtype, p->k_dtype, p->heads, p->dim, p->batch, p->n_q, 1,
                          nullptr, rows, false, topk, out_idx, st, flt);
}

int32_t idx_score_topk_static(const idx_problem* p, int32_t topk, int32_t* out_idx, float* out_scores,
                              void* stream) {
  static_assert(IDX_STATIC_SCRATCH_BYTES == kStaticScratchBytes, "header and library scratch sizes agree");
  int rc = check_problem(p);
  if (rc != IDX_OK) return rc;
  if (topk < 1 || !out_idx) return IDX_EINVAL;
  if (idx_workspace_bytes(p, IDX_OP_SCORE_TOPK, 0, 0, topk) > kStaticScratchBytes) return IDX_ETOOLARGE;
  void* scratch = nullptr;
  if (static_scratch_ptr(&scratch) != hipSuccess) return IDX_EHIP;
  return idx_score_topk(p, topk, out_idx, out_scores, scratch, kStaticScratchBytes, stream);
}

int32_t idx_group_proxy_scan(const idx_problem* p, int32_t group, int32_t n_cand,
                             int32_t* out_cand, void* out_proxy_q, float* out_proxy_w,
                             float* out_proxy_scores, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != IDX_OK) return rc;
  if (group < 1 || n_cand < 1 || !out_cand) return IDX_EINVAL;
  const int pqf = proxy_q_dtype(p);
  if (!combo_supported(pqf, p->k_dtype, p->heads, p->dim)) return IDX_EUNSUPPORTED;
  const size_t need = idx_workspace_bytes(p, IDX_OP_GROUP_PROXY_SCAN, group, n_cand, 0);
  if (!ws || ws_bytes < need) return IDX_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int n_g = ceil_div(p->n_q, group);
  char* cur = (char*)ws;
  void* pq = out_proxy_q ? out_proxy_q : (void*)cur;
  cur += align_up(proxy_q_bytes(p, n_g));
  float* pw = out_proxy_w ? out_proxy_w : (float*)cur;
  cur += align_up((size_t)p->batch * n_g * p->heads * 4);
  if (timed(IDX_KERNEL_PROXY, st, [&] {
        return launch_proxy_build(p->q, p->q_scale, p->w, p->batch, p->n_q, p->heads, p->dim,
                                  p->q_dtype, group, pq, pw, st);
      }) != hipSuccess)
    return IDX_EHIP;
  const bool full = out_proxy_scores != nullptr;
  if (split_shape(p, n_g, pqf)) {
    if (full && timed(IDX_KERNEL_FILL, st, [&] {
          return launch_fill(out_proxy_scores, (size_t)p->batch * n_g * p->n_k, -__builtin_huge_valf(), st);
        }) != hipSuccess)
      return IDX_EHIP;
    return split_score_select(p, pqf, pq, nullptr, pw, n_g, kModeProxy, group, 1, n_cand, out_cand,
                              out_proxy_scores, cur, st);
  }
  Layout L = make_layout(kModeProxy, p, n_g, p->n_k, group);
  float* buf;
  long long rows;
  if (full) {
    buf = out_proxy_scores;
    rows = (long long)p->batch * n_g;
    if (timed(IDX_KERNEL_FILL, st, [&] {
          return launch_fill(buf, (size_t)rows * p->n_k, -__builtin_huge_valf(), st);
        }) != hipSuccess)
      return IDX_EHIP;
  } else {
    buf = (float*)cur;
    rows = (long long)((ws_bytes - (size_t)(cur - (char*)ws)) / ((size_t)p->n_k * 4));
  }
  ScoreArgs sa = base_args(p);
  sa.q = pq;
  sa.q_scale = nullptr;
  sa.w = pw;
  sa.n_rows = n_g;
  sa.group = group;
  sa.mode = kModeProxy;
  return score_and_select(sa, L, pqf, p->k_dtype, p->heads, p->dim, p->batch, p->n_q, group, buf,
                          rows, full, n_cand, out_cand, st);
}

int32_t idx_refine_topk(const idx_problem* p, int32_t group, const int32_t* cand, int32_t n_cand,
                        int32_t topk, int32_t* out_idx, float* out_cand_scores, void* ws,
                        size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != IDX_OK) return rc;
  if (group < 1 || n_cand < 1 || topk < 1 || !cand || !out_idx) return IDX_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  Layout L = make_layout(kModeGather, p, p->n_q, n_cand, group);
  const bool full = out_cand_scores != nullptr;
  float* buf;
  int* recs = nullptr;  // the rows' boundary records (workspace path only)
  long long rows;
  if (full) {
    buf = out_cand_scores;
    rows = (long long)p->batch * p->n_q;
  } else {
    const size_t need = idx_workspace_bytes(p, IDX_OP_REFINE_TOPK, group, n_cand, topk);
    if (!ws || ws_bytes < need) return IDX_EWORKSPACE;
    rows = buffer_rows(L, (long long)p->batch * p->n_q);
    buf = (float*)ws;
    recs = (int*)((char*)ws + align_up((size_t)rows * n_cand * 4));
  }
  ScoreArgs sa = base_args(p);
  sa.group = group;
  sa.n_cols = n_cand;
  sa.cand = cand;
  sa.mode = kModeGather;
  return score_and_select(sa, L, p->q_dtype, p->k_dtype, p->heads, p->dim, p->batch, p->n_q,
                          group, buf, rows, full, topk, out_idx, st, Filter(), recs);
}

int32_t idx_reuse_topk(const idx_problem* p, int32_t group, const int32_t* proxy_topk,
                       int32_t topk, int32_t* out_idx, void* stream) {
  if (!p || p->batch < 1 || p->n_q < 1 || p->n_k < 1) return IDX_EINVAL;
  if (p->q_pos0 < 0 || (long long)p->q_pos0 + p->n_q > p->n_k) return IDX_EINVAL;
  if (group < 1 || topk < 1 || !proxy_topk || !out_idx) return IDX_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (timed(IDX_KERNEL_REUSE, st, [&] {
        return launch_reuse(proxy_topk, p->batch, p->n_q, p->q_pos0, group, topk, out_idx, st);
      }) != hipSuccess)
    return IDX_EHIP;
  return IDX_OK;
}

int32_t idx_block_route(const idx_problem* p, int32_t group, int32_t block, int32_t n_sel,
                        int32_t* out_cand, void* out_block_means, float* out_block_scores,
                        void* out_proxy_q, float* out_proxy_w, void* ws, size_t ws_bytes,
                        void* stream) {
  int rc = check_problem(p);
  if (rc != IDX_OK) return rc;
  if (group < 1 || block < 1 || n_sel < 1 || !out_cand) return IDX_EINVAL;
  if ((long long)(n_sel + 1) * block > 0x7FFFFFFF) return IDX_EINVAL;
  const BlockLayout BL = block_layout(p, group, block, n_sel);
  if (!ws || ws_bytes < BL.total) return IDX_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int n_g = ceil_div(p->n_q, group);
  char* base = (char*)ws;
  void* pq = out_proxy_q ? out_proxy_q : (void*)(base + BL.pq);
  float* pw = out_proxy_w ? out_proxy_w : (float*)(base + BL.pw);
  void* kbar = out_block_means ? out_block_means : (void*)(base + BL.kbar);
  int* sel = (int*)(base + BL.sel);
  if (timed(IDX_KERNEL_PROXY, st, [&] {
        hipError_t e = launch_proxy_build(p->q, p->q_scale, p->w, p->batch, p->n_q, p->heads, p->dim,
                                          p->q_dtype, group, pq, pw, st);
        return e != hipSuccess ? e
                               : launch_block_means(p->k, p->k_scale, p->batch, p->n_k, p->dim, p->k_dtype,
                                                    block, kbar, st);
      }) != hipSuccess)
    return IDX_EHIP;
  const idx_problem q = block_problem(p, block, pq, pw, kbar);
  const bool full = out_block_scores != nullptr;
  if (full && timed(IDX_KERNEL_FILL, st, [&] {
        return launch_fill(out_block_scores, (size_t)p->batch * n_g * q.n_k, -__builtin_huge_valf(), st);
      }) != hipSuccess)
    return IDX_EHIP;
  if (BL.split) {
    rc = split_score_select(&q, q.q_dtype, pq, nullptr, pw, n_g, kModeBlock, group, block, n_sel, sel,
                            out_block_scores, base + BL.scan, st);
  } else {
    Layout L = make_layout(kModeBlock, &q, n_g, q.n_k, group);
    ScoreArgs sa = base_args(&q);
    sa.n_rows = n_g;
    sa.group = group;
    sa.block = block;
    sa.mode = kModeBlock;
    float* buf = full ? out_block_scores : (float*)(base + BL.scan);
    const long long rows = full ? (long long)p->batch * n_g : BL.rows;
    rc = score_and_select(sa, L, q.q_dtype, q.k_dtype, p->heads, p->dim, p->batch, p->n_q, group, buf,
                          rows, full, n_sel, sel, st);
  }
  if (rc != IDX_OK) return rc;
  if (timed(IDX_KERNEL_REUSE, st, [&] {
        return launch_block_expand(sel, p->batch, p->n_q, p->q_pos0, group, block, n_sel, out_cand, st);
      }) != hipSuccess)
    return IDX_EHIP;
  return IDX_OK;
}

int32_t idx_ivf_build(const idx_problem* p, int32_t n_clusters, int32_t refit, int32_t iters,
                      void* out_centroids, int32_t* out_offsets, int32_t* out_members, int32_t* out_counts,
                      int32_t* out_assign, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_keys(p);
  if (rc != IDX_OK) return rc;
  const int m = n_clusters, R = refit;
  if (!ivf_params_ok(m, R) || iters < 0 || iters > 64) return IDX_EINVAL;
  const int n_v = p->n_k / R;
  if (n_v == 0) return IDX_OK;  // no refit point inside the keys: the outputs are empty
  if (!out_centroids || !out_offsets || !out_members || !out_counts) return IDX_EINVAL;
  const IvfBuildLayout L = ivf_build_layout(p, m);
  if (!ws || ws_bytes < L.total) return IDX_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  const int B = p->batch, n_k = p->n_k, D = p->dim, kf = p->k_dtype, nt = ivf_tiles(n_k);
  const size_t eb = ivf_cent_elt(p);
  const long long cent_bs = (long long)n_v * m * D, offs_bs = (long long)n_v * (m + 1);
  const long long mem_bs = (long long)n_v * n_k, cnt_bs = (long long)n_v * (nt + 1) * m;
  auto version_cent = [&](int u) { return (void*)((char*)out_centroids + (size_t)(u - 1) * m * D * eb); };

  // One assignment pass over keys [0, n) with centroids (cent, bs) into the
  // given lists (published when `pub` >= 1: that version's slots).
  auto pass = [&](const void* cent, long long cbs, int n, int pub) {
    IvfPassArgs a = {};
    a.k = p->k;
    a.k_scale = p->k_scale;
    a.n_k = n_k;
    a.m = m;
    a.n_assign = n;
    a.cent = cent;
    a.cent_bs = cbs;
    a.rank = (int*)(base + L.rank);
    a.rank_bs = n_k;
    a.tilecnt = (int*)(base + L.tilecnt);
    a.tilecnt_bs = (long long)nt * m;
    if (pub >= 1) {
      a.assign = out_assign ? out_assign + (size_t)(pub - 1) * n_k : (int*)(base + L.assign);
      a.assign_bs = out_assign ? mem_bs : n_k;
      a.counts = out_counts + (size_t)(pub - 1) * (nt + 1) * m;
      a.counts_bs = cnt_bs;
      a.offsets = out_offsets + (size_t)(pub - 1) * (m + 1);
      a.offsets_bs = offs_bs;
      a.members = out_members + (size_t)(pub - 1) * n_k;
      a.members_bs = mem_bs;
    } else {
      a.assign = (int*)(base + L.assign);
      a.assign_bs = n_k;
      a.counts = (int*)(base + L.counts);
      a.counts_bs = (long long)(nt + 1) * m;
      a.offsets = (int*)(base + L.offsets);
      a.offsets_bs = m + 1;
      a.members = (int*)(base + L.members);
      a.members_bs = n_k;
    }
    return launch_ivf_pass(a, kf, D, B, st);
  };
  auto update = [&](const void* src, long long sbs, void* dst, const int* offs, long long obs, const int* mem,
                    long long mbs, int copy_only) {
    IvfUpdateArgs a = {};
    a.k = p->k;
    a.k_scale = p->k_scale;
    a.n_k = n_k;
    a.m = m;
    a.copy_only = copy_only;
    a.offsets = offs;
    a.offsets_bs = obs;
    a.members = mem;
    a.members_bs = mbs;
    a.src = src;
    a.src_bs = sbs;
    a.dst = dst;
    a.dst_bs = cent_bs;
    return launch_ivf_update(a, kf, D, B, st);
  };

  return timed(IDX_KERNEL_IVF_BUILD, st, [&]() -> hipError_t {
    hipError_t e = hipSuccess;
    if (out_assign) {
      e = launch_fill_i32(out_assign, (size_t)B * n_v * n_k, -1, st);
      if (e != hipSuccess) return e;
    }
    e = launch_ivf_init(p->k, p->k_scale, kf, B, n_k, D, m, R, base + L.cur, (long long)m * D, st);
    if (e != hipSuccess) return e;
    const void* prev = base + L.cur;
    long long prev_bs = (long long)m * D;
    for (int u = 1; u <= n_v; ++u) {
      void* dst = version_cent(u);
      for (int it = 0; it < iters; ++it) {
        const void* src = it == 0 ? prev : dst;
        const long long sbs = it == 0 ? prev_bs : cent_bs;
        if (it == 0 && u > 1) {
          // the lists published for version u-1 are the assignment of keys
          // [0, u R) to its centroids: this iteration's assignment
          e = update(src, sbs, dst, out_offsets + (size_t)(u - 2) * (m + 1), offs_bs,
                     out_members + (size_t)(u - 2) * n_k, mem_bs, 0);
        } else {
          e = pass(src, sbs, u * R, 0);
          if (e == hipSuccess)
            e = update(src, sbs, dst, (int*)(base + L.offsets), m + 1, (int*)(base + L.members), n_k, 0);
        }
        if (e != hipSuccess) return e;
      }
      if (iters == 0) {
        e = update(prev, prev_bs, dst, (int*)(base + L.offsets), m + 1, (int*)(base + L.members), n_k, 1);
        if (e != hipSuccess) return e;
      }
      e = pass(dst, cent_bs, std::min((long long)(u + 1) * R, (long long)n_k), u);
      if (e != hipSuccess) return e;
      prev = dst;
      prev_bs = cent_bs;
    }
    return hipSuccess;
  }) != hipSuccess ? IDX_EHIP : IDX_OK;
}

int32_t idx_ivf_route(const idx_problem* p, int32_t group, int32_t n_clusters, int32_t refit,
                      int32_t insert_batch, int32_t n_cand, const void* centroids, const int32_t* offsets,
                      const int32_t* members, const int32_t* counts, int32_t* out_cand,
                      float* out_cluster_scores, void* out_proxy_q, float* out_proxy_w, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = check_problem(p);
  if (rc != IDX_OK) return rc;
  const int m = n_clusters, R = refit;
  if (group < 1 || !ivf_params_ok(m, R) || !out_cand) return IDX_EINVAL;
  if (insert_batch < kIvfTile || insert_batch % kIvfTile != 0 || insert_batch > R || n_cand < R) return IDX_EINVAL;
  const int n_v = p->n_k / R;
  if (n_v >= 1 && (!centroids || !offsets || !members || !counts)) return IDX_EINVAL;
  const int pqf = proxy_q_dtype(p);
  if (!combo_supported(pqf, ivf_cent_dtype(p), p->heads, p->dim)) return IDX_EUNSUPPORTED;
  const IvfRouteLayout L = ivf_route_layout(p, group, m);
  if (!ws || ws_bytes < L.total) return IDX_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  const int n_g = ceil_div(p->n_q, group);
  void* pq = out_proxy_q ? out_proxy_q : (void*)(base + L.pq);
  float* pw = out_proxy_w ? out_proxy_w : (float*)(base + L.pw);
  if (timed(IDX_KERNEL_PROXY, st, [&] {
        return launch_proxy_build(p->q, p->q_scale, p->w, p->batch, p->n_q, p->heads, p->dim, p->q_dtype,
                                  group, pq, pw, st);
      }) != hipSuccess)
    return IDX_EHIP;
  IvfRouteArgs a = {};
  a.pq = pq;
  a.pw = pw;
  a.cents = centroids;
  a.offsets = offsets;
  a.members = members;
  a.counts = counts;
  a.n_v = n_v;
  a.m = m;
  a.n_k = p->n_k;
  a.n_tiles = ivf_tiles(p->n_k);
  a.n_g = n_g;
  a.n_q = p->n_q;
  a.q_pos0 = p->q_pos0;
  a.group = group;
  a.refit = R;
  a.batch = insert_batch;
  a.n_cand = n_cand;
  a.scores = out_cluster_scores ? out_cluster_scores : (float*)(base + L.scores);
  a.cand = out_cand;
  if (timed(IDX_KERNEL_IVF_ROUTE, st, [&] {
        return launch_ivf_route(a, pqf, p->heads, p->dim, p->batch, st);
      }) != hipSuccess)
    return IDX_EHIP;
  return IDX_OK;
}

int32_t idx_profile_enable(int32_t on) {
  g_profile = on != 0;
  return IDX_OK;
}

int32_t idx_profile_read(float* ms, int32_t* launches) {
  int rc = IDX_OK;
  for (int i = 0; i < IDX_KERNEL_KINDS; ++i) {
    if (ms) ms[i] = 0.f;
    if (launches) launches[i] = 0;
  }
  for (const TimedLaunch& r : g_records) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
      rc = IDX_EHIP;
    if (r.kind >= 0 && r.kind < IDX_KERNEL_KINDS) {
      if (ms) ms[r.kind] += t;
      if (launches) launches[r.kind] += 1;
    }
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_records.clear();
  return rc;
}

}  // extern "C"
