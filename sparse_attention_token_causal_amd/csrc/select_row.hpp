// Per-row exact top-k select for gfx950 (the device function; select.hip
// launches it one workgroup per row, split.hip once per decode row).
//
// One workgroup per row of scores.  The order is (score descending, key
// index ascending) with exact equality as a tie and -0 == +0 ("PIVOT:
// Efficient Query-Group Indexing for Token-Level Sparse Attention",
// Abstract: each query keeps its own top-k of the scanned or re-scored
// keys; the tie rule is the reading given in the library header).
//
// Method (scores are mapped to order-preserving 32-bit keys):
//  1. load the row (into registers when it is short enough, coalesced) and
//     reduce the count, minimum and maximum of the eligible keys;
//  2. all eligible keys share the bits above the highest bit where min and
//     max differ, so one 2048-bin histogram of the next 11 bits spreads the
//     row; a suffix scan finds the bin b* holding the k-th key;
//  3. every key in a bin above b* is a winner; the keys of b* are gathered
//     into an LDS list and ranked exactly by counting how many list entries
//     precede each one in (key desc, index asc) order; the first `need`
//     ranks win (ties need no second pass: the index is part of the order);
//     while the boundary bin is larger than the list, the histogram step is
//     repeated on the next 11 bits inside it (an MSB-first radix descent); a
//     class of equal keys larger than the list is split by an ascending radix
//     select over the key indices;
//  4. winners are written with one block-wide prefix scan of per-thread
//     counts (the row is a set; the order is fixed by the thread layout),
//     the boundary winners at their rank, and the row is padded with -1.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace idx {

constexpr int kBins = 2048;
constexpr int kListCap = 2048;  // LDS list capacity
constexpr int kRankMax = 256;   // descend until the boundary bin is at most this large
constexpr int kMaxNW = 1024 / kWave;

struct SelectShared {
  uint32_t hist[kBins];
  uint32_t lkey[kListCap];
  int lidx[kListCap];
  int wred[3][kMaxNW];
  int wscan[kMaxNW];
  int list_n;
  int out_n;  // output slots reserved (the streaming variant's last pass)
  uint32_t sel_bin;
  int sel_above;
  // fallback radix state
  uint32_t bins256[256];
  int soff[kMaxSegs + 1];  // segmented lists: offset of each segment in the gathered list
};

__device__ __forceinline__ int row_length(const SelectArgs& a, int r, unsigned blk) {
  if (a.mode == kModeList)
    return min(a.finfo ? a.finfo[kFiltInfoStride * (long long)blk + kFiltInfoCount] : a.counts[blk],
               a.n_cols);
  if (a.mode == kModeGather) return a.n_cols;
  const int lim = mode_limit(a.mode, a.q_pos0, a.n_q, a.group, a.block, r);
  return min(lim + 1, a.n_cols);
}

__device__ __forceinline__ uint32_t load_key(const float* row, int c) {
  const float v = row[c];
  return v == neg_inf() ? kKeyExcluded : order_key(v);
}

// Wave inclusive prefix sum with shuffles.  The select keeps this form
// rather than the DPP one of the other kernels: with the DPP form the
// register allocation of the 32-keys-per-thread variant (bounded to 128
// VGPRs) spills the gathered rows' key indices during the row load and
// serializes those loads, which made the Refine selects 14% slower.
__device__ __forceinline__ int wave_incl_scan_shfl(int v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (l >= off) v += o;
  }
  return v;
}

// Block-wide exclusive scan of one int per thread; also returns the total.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* total, SelectShared& sh) {
  constexpr int kNW = NT / kWave;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int incl = wave_incl_scan_shfl(v);
  if (lane == kWave - 1) sh.wscan[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kNW; ++i) {
    const int s = sh.wscan[i];
    before += (i < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

// NT threads per row; blk is the row within the launch.  KPT > 0: each
// thread keeps the keys of columns tid + i*NT (i < KPT) in registers.
// KPT == 0: rows of any length, re-read from global memory in batches of 8
// loads per thread.  (Rows whose scan left a record take the one-pass
// select of select.hip first; this is their general path.)
// A row's select is a chain of short dependent phases (loads, reductions,
// histogram, scans), so rows in flight per CU decide its speed: 256-thread
// workgroups are held to at least four waves per SIMD (at most 128 VGPRs,
// four rows per CU; the LDS would allow five).
template <int NT, int KPT>
__device__ __forceinline__ void select_row(const SelectArgs& a, const unsigned blk, SelectShared& sh) {
  constexpr int kSelectThreads = NT;
  constexpr int kNW = NT / kWave;
  const long long frow = a.row0 + blk;
  const int b = (int)(frow / a.n_rows), r = (int)(frow % a.n_rows);
  const float* row = a.scores + (long long)blk * a.ld;
  int* out = a.out + frow * (long long)a.topk;
  const int* crow = nullptr;
  if (a.mode == kModeGather) {
    const int n_g = (a.n_q + a.group - 1) / a.group;
    crow = a.cand + ((long long)b * n_g + r / a.group) * a.n_cols;
  }
  if (a.mode == kModeList) crow = a.lidx + (long long)blk * a.ld;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  int len;
  if (a.mode == kModeList && a.seg_counts) {
    // Segmented list: segment s of the row holds seg_counts[s] entries from
    // position s * seg_len.  Gather them, in segment order, into one
    // contiguous list (gval/gidx) that the rest of the kernel reads.
    const int ns = a.n_segs;
    int tot;
    const int cnt = tid < ns ? a.seg_counts[(long long)blk * ns + tid] : 0;
    const int ex = block_excl_scan<NT>(cnt, &tot, sh);
    if (tid < ns) sh.soff[tid] = ex;
    if (tid == 0) sh.soff[ns] = tot;
    __syncthreads();
    float* gv = a.gval + (long long)blk * a.ld;
    int* gi = a.gidx + (long long)blk * a.ld;
    for (int c0 = 0; c0 < tot; c0 += 8 * NT) {
      float v[8];
      int x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = min(c0 + j * NT + tid, tot - 1);
        int lo = 0, hi = ns - 1;  // last segment whose offset is <= c
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sh.soff[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const long long src = (long long)lo * a.seg_len + (c - sh.soff[lo]);
        v[j] = row[src];
        x[j] = crow[src];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = c0 + j * NT + tid;
        if (c < tot) {
          gv[c] = v[j];
          gi[c] = x[j];
        }
      }
    }
    __syncthreads();
    row = gv;
    crow = gi;
    len = min(tot, a.n_cols);
  } else {
    len = row_length(a, r, blk);
  }
  constexpr int REG = KPT > 0 ? KPT : 1;
  uint32_t keys[REG];
  // rows longer than the register tile (possible for candidate lists) stream
  const bool regs = KPT > 0 && len <= REG * kSelectThreads;

  // Rows with their own key indices (gather, list) keep the indices beside the
  // keys (registers, or batched loads when streaming): no dependent loads
  // later.  Otherwise the key index is the column.
  const bool indexed = crow != nullptr;
  int idxs[REG];
  auto key_at = [&](int c) -> uint32_t { return load_key(row, c); };
  // Calls f(column, key, key index) for every column of this thread (eligible or not).
  auto for_keys = [&](auto&& f) {
    if (KPT > 0 && regs) {
#pragma unroll
      for (int i = 0; i < REG; ++i) {
        const int c = i * kSelectThreads + tid;
        f(c, keys[i], indexed ? idxs[i] : c);
      }
    } else {
      for (int c0 = 0; c0 < len; c0 += 8 * kSelectThreads) {
        float v[8];
        int x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int cc = min(c0 + j * kSelectThreads + tid, max(len - 1, 0));
          v[j] = row[cc];
          x[j] = indexed ? crow[cc] : cc;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = c0 + j * kSelectThreads + tid;
          f(c, (c < len && v[j] != neg_inf()) ? order_key(v[j]) : kKeyExcluded, x[j]);
        }
      }
    }
  };

  // ---- 1. load (batched, clamped addresses), count, min, max ----
  int nv = 0;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if (KPT > 0 && regs) {
    // every load of the row at once (clamped addresses: no per-element branch)
    float v[REG];
#pragma unroll
    for (int i = 0; i < REG; ++i) {
      const int cc = min(i * kSelectThreads + tid, max(len - 1, 0));
      v[i] = row[cc];
      if (indexed) idxs[i] = crow[cc];
    }
#pragma unroll
    for (int i = 0; i < REG; ++i) {
      const int c = i * kSelectThreads + tid;
      keys[i] = (c < len && v[i] != neg_inf()) ? order_key(v[i]) : kKeyExcluded;
    }
  }
  // count, minimum and maximum of the eligible keys that `visit` passes to
  // its callback, reduced over the workgroup
  int n_valid = 0;
  auto key_stats = [&](auto&& visit) {
    nv = 0;
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
    visit([&](uint32_t k) {
      if (k != kKeyExcluded) {
        ++nv;
        kmin = min(kmin, k);
        kmax = max(kmax, k);
      }
    });
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nv += __shfl_xor(nv, off, kWave);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off, kWave));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off, kWave));
    }
    if (lane == 0) {
      sh.wred[0][wave] = nv;
      sh.wred[1][wave] = (int)kmin;
      sh.wred[2][wave] = (int)kmax;
    }
    __syncthreads();
    n_valid = 0;
    kmin = 0xFFFFFFFFu;
    kmax = 0u;
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
      n_valid += sh.wred[0][i];
      kmin = min(kmin, (uint32_t)sh.wred[1][i]);
      kmax = max(kmax, (uint32_t)sh.wred[2][i]);
    }
    __syncthreads();
  };
  // Linear bins over [kmin, kmax] (section 2a) spread the row's values when
  // this holds.
  auto spreads = [&](uint32_t lo, uint32_t hi) {
    const float vlo = key_to_float(lo), vhi = key_to_float(hi);
    const float scale = (float)(kBins - 1) / (vhi - vlo);
    return vhi > vlo && scale > 0.f && scale < __builtin_huge_valf();
  };
  // A streamed row takes the range of its linear bins from a sample (16
  // evenly spaced runs of 256 columns) instead of a pass over the row: keys
  // outside the sample's range fall in the edge bins (the map stays
  // monotone), each bin's exact key range is still recorded, and the bins'
  // total is the row's count of eligible keys.  A sample without spread
  // falls back to the pass.
  bool sampled = false;
  if constexpr (KPT == 0) {
    constexpr int kRun = 256, kRuns = 16;
    if (len >= 2 * kRun * kRuns) {
      key_stats([&](auto&& f) {
        for (int i = tid; i < kRun * kRuns; i += kSelectThreads) {
          const int c = (int)((long long)(i / kRun) * len / kRuns) + i % kRun;
          const float v = row[c];
          f(v != neg_inf() ? order_key(v) : kKeyExcluded);
        }
      });
      // (workgroup-wide values only: the branch below holds barriers)
      sampled = n_valid > 0 && spreads(kmin, kmax);
    }
  }
  if (!sampled) key_stats([&](auto&& f) { for_keys([&](int, uint32_t k, int) { f(k); }); });
  const int topk = a.topk;
  int kk = min(topk, n_valid);

  // ---- 2. narrow the boundary interval [blo, bhi] of keys ----
  // `above` eligible keys lie above the interval and `need` of the keys inside
  // it still win.  Winners = keys above the interval, plus either all of it
  // or its `need` best entries in (key desc, index asc) order.
  uint32_t blo = kmin, bhi = kmax;
  int above = 0, need = kk, in_bin = n_valid;
  bool idx_radix = false, gather_late = false;
  int idx_thr = 0;

  // Suffix scan over the histogram: picks the bin holding rank `need`
  // (descending); returns the bin, and the count above it via *before.
  auto pick_desc = [&](int* before_out) -> uint32_t {
    constexpr int BPT = kBins / NT;
    int cnt[BPT], s = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      cnt[j] = (int)sh.hist[kBins - 1 - (BPT * tid + j)];
      s += cnt[j];
    }
    int total;
    int before = block_excl_scan<NT>(s, &total, sh);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (before < need && need <= before + cnt[j]) {
        sh.sel_bin = (uint32_t)(kBins - 1 - (BPT * tid + j));
        sh.sel_above = before;
      }
      before += cnt[j];
    }
    __syncthreads();
    *before_out = sh.sel_above;
    return sh.sel_bin;
  };

  if (sampled || n_valid > topk) {
    // 2a. one pass of 2048 bins linear in the score value between the row's
    // minimum and maximum (a monotone map: a larger score never lands in a
    // lower bin), which spreads the bulk of a row over many bins
    const float vlo = key_to_float(blo), vhi = key_to_float(bhi);
    const float scale = (float)(kBins - 1) / (vhi - vlo);
    if (spreads(blo, bhi)) {
      const float off = -vlo * scale;
      auto lbin = [&](uint32_t k) {
        const float x = __builtin_fmaf(key_to_float(k), scale, off);
        return (uint32_t)min(max((int)x, 0), kBins - 1);
      };
      // (KPT == 0: each bin's key range is kept in the list arrays during
      // the same pass, so the row is not read again for it)
      static_assert(kListCap >= kBins, "a key range per bin");
      for (int i = tid; i < kBins; i += kSelectThreads) {
        sh.hist[i] = 0;
        if constexpr (KPT == 0) {
          sh.lkey[i] = 0xFFFFFFFFu;
          sh.lidx[i] = 0;
        }
      }
      __syncthreads();
      for_keys([&](int, uint32_t k, int) {
        if (k != kKeyExcluded) {
          const uint32_t bn = lbin(k);
          atomicAdd(&sh.hist[bn], 1u);
          if constexpr (KPT == 0) {
            atomicMin(&sh.lkey[bn], k);
            atomicMax((uint32_t*)&sh.lidx[bn], k);
          }
        }
      });
      __syncthreads();
      if (sampled) {
        // the row's count of eligible keys; with at most topk of them every
        // one wins: the whole key range is the (whole) boundary interval
        constexpr int BPT = kBins / NT;
        int s_ = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) s_ += (int)sh.hist[BPT * tid + j];
        block_excl_scan<NT>(s_, &n_valid, sh);
        kk = min(topk, n_valid);
        need = kk;
        in_bin = n_valid;
        if (n_valid <= topk) {
          blo = 1u;  // every eligible key (the excluded key is 0)
          bhi = 0xFFFFFFFFu;
        }
      }
      if (!sampled || n_valid > topk) {
      int before;
      const uint32_t b = pick_desc(&before);
      above += before;
      need -= before;
      in_bin = (int)sh.hist[b];
      if constexpr (KPT == 0) {
        blo = sh.lkey[b];
        bhi = (uint32_t)sh.lidx[b];
        __syncthreads();
      } else {
      // the key range of that bin
      uint32_t mn = 0xFFFFFFFFu, mx = 0u;
      for_keys([&](int, uint32_t k, int) {
        if (k != kKeyExcluded && lbin(k) == b) {
          mn = min(mn, k);
          mx = max(mx, k);
        }
      });
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
      }
      if (lane == 0) {
        sh.wred[1][wave] = (int)mn;
        sh.wred[2][wave] = (int)mx;
      }
      __syncthreads();
      blo = 0xFFFFFFFFu;
      bhi = 0u;
#pragma unroll
      for (int i = 0; i < kNW; ++i) {
        blo = min(blo, (uint32_t)sh.wred[1][i]);
        bhi = max(bhi, (uint32_t)sh.wred[2][i]);
      }
      __syncthreads();
      }
      }
    }
    // 2b. MSB-first radix descent in 11-bit digits inside [blo, bhi]
    while (in_bin > kRankMax && blo != bhi && in_bin != need) {
      const uint32_t diff = blo ^ bhi;
      const int S = 32 - __builtin_clz(diff);  // bits >= S are shared by the interval
      const int w = S < 11 ? S : 11;
      const int shift = S - w;
      const uint32_t dmask = (1u << w) - 1u;
      for (int i = tid; i < kBins; i += kSelectThreads) sh.hist[i] = 0;
      __syncthreads();
      const uint32_t lo = blo, hi = bhi;
      for_keys([&](int, uint32_t k, int) {
        if (k != kKeyExcluded && k >= lo && k <= hi) atomicAdd(&sh.hist[(k >> shift) & dmask], 1u);
      });
      __syncthreads();
      int before;
      const uint32_t d = pick_desc(&before);
      above += before;
      need -= before;
      in_bin = (int)sh.hist[d];
      const uint32_t base = S >= 32 ? 0u : (lo >> S) << S;
      const uint32_t dlo = base | (d << shift);
      const uint32_t dhi = dlo + ((1u << shift) - 1u);
      blo = max(blo, dlo);
      bhi = min(bhi, dhi);
      __syncthreads();
    }
    if (in_bin != need) {
      if (KPT == 0 && in_bin <= kListCap) {
        gather_late = true;  // in the streaming variant's single last pass
      } else if (in_bin <= kListCap) {
        // ---- 3. gather the boundary interval and rank it exactly ----
        if (tid == 0) sh.list_n = 0;
        __syncthreads();
        const uint32_t lo = blo, hi = bhi;
        for_keys([&](int, uint32_t k, int ix) {
          if (k != kKeyExcluded && k >= lo && k <= hi) {
            const int slot = atomicAdd(&sh.list_n, 1);
            sh.lkey[slot] = k;
            sh.lidx[slot] = ix;
          }
        });
        __syncthreads();
        const int m = sh.list_n;
        for (int i = tid; i < m; i += kSelectThreads) {
          const uint32_t ki = sh.lkey[i];
          const int xi = sh.lidx[i];
          int rank = 0;
          for (int j = 0; j < m; ++j) {
            const uint32_t kj = sh.lkey[j];
            rank += (kj > ki) || (kj == ki && sh.lidx[j] < xi);
          }
          if (rank < need) out[above + rank] = xi;
        }
      } else {
        // blo == bhi: a class of more than kListCap equal keys; `need` of them
        // win by smallest key index (ascending radix over the indices)
        idx_radix = true;
        const uint32_t tau = blo;
        uint32_t ip = 0, im = 0;
        int rank = need;
        for (int shift = 24; shift >= 0; shift -= 8) {
          for (int i = tid; i < 256; i += kSelectThreads) sh.bins256[i] = 0;
          __syncthreads();
          for_keys([&](int, uint32_t k, int ixv) {
            if (k == tau) {
              const uint32_t ix = (uint32_t)ixv;
              if ((ix & im) == ip) atomicAdd(&sh.bins256[(ix >> shift) & 255u], 1u);
            }
          });
          __syncthreads();
          if (tid == 0) {
            int below = 0;
            for (int d = 0; d < 256; ++d) {
              const int n = (int)sh.bins256[d];
              if (below + n >= rank) {
                sh.sel_bin = (uint32_t)d;
                sh.sel_above = below;
                break;
              }
              below += n;
            }
          }
          __syncthreads();
          rank -= sh.sel_above;
          ip |= sh.sel_bin << shift;
          im |= 255u << shift;
          __syncthreads();
        }
        idx_thr = (int)ip;
      }
    }
  }
  const bool whole = in_bin == need;

  // ---- 4. compaction: keys above the interval (and all of it when it all wins) ----
  const uint32_t cut_hi = bhi, cut_lo = blo;
  auto certain = [&](uint32_t k) -> bool {
    return k != kKeyExcluded && (k > cut_hi || (whole && k >= cut_lo));
  };
  if constexpr (KPT == 0) {
    if (!idx_radix) {
      // one pass over the row: the winners above the interval go to the
      // output at slots reserved once per wave and batch (a row is a set),
      // and the interval's keys, when they are ranked, to the LDS list
      if (tid == 0) {
        sh.list_n = 0;
        sh.out_n = 0;
      }
      __syncthreads();
      for (int c0 = 0; c0 < len; c0 += 8 * kSelectThreads) {
        float v[8];
        int x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int cc = min(c0 + j * kSelectThreads + tid, max(len - 1, 0));
          v[j] = row[cc];
          x[j] = indexed ? crow[cc] : cc;
        }
        uint32_t cm = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = c0 + j * kSelectThreads + tid;
          const uint32_t k = (c < len && v[j] != neg_inf()) ? order_key(v[j]) : kKeyExcluded;
          cm |= (uint32_t)certain(k) << j;
          if (gather_late && k != kKeyExcluded && k >= cut_lo && k <= cut_hi) {
            const int slot = atomicAdd(&sh.list_n, 1);
            sh.lkey[slot] = k;
            sh.lidx[slot] = x[j];
          }
        }
        const int n = __builtin_popcount(cm);
        const int incl = wave_incl_scan(n);
        const int wt = __builtin_amdgcn_readlane(incl, kWave - 1);
        int base = 0;
        if (lane == kWave - 1 && wt) base = atomicAdd(&sh.out_n, wt);
        int pos = __builtin_amdgcn_readlane(base, kWave - 1) + incl - n;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((cm >> j) & 1u) out[pos++] = x[j];
      }
      if (gather_late) {
        __syncthreads();
        const int m = sh.list_n;
        for (int i = tid; i < m; i += kSelectThreads) {
          const uint32_t ki = sh.lkey[i];
          const int xi = sh.lidx[i];
          int rank = 0;
          for (int j = 0; j < m; ++j) {
            const uint32_t kj = sh.lkey[j];
            rank += (kj > ki) || (kj == ki && sh.lidx[j] < xi);
          }
          if (rank < need) out[above + rank] = xi;
        }
      }
      for (int i = kk + tid; i < topk; i += kSelectThreads) out[i] = -1;
      return;
    }
  }
  int mine = 0;
  for_keys([&](int, uint32_t k, int) { mine += certain(k); });
  int total;
  int off = block_excl_scan<NT>(mine, &total, sh);
  for_keys([&](int, uint32_t k, int ix) {
    if (certain(k)) out[off++] = ix;
  });
  if (idx_radix) {
    const uint32_t tau = blo;
    int tmine = 0;
    for_keys([&](int, uint32_t k, int ix) { tmine += (k == tau && ix <= idx_thr); });
    int ttot;
    int toff = above + block_excl_scan<NT>(tmine, &ttot, sh);
    for_keys([&](int, uint32_t k, int ix) {
      if (k == tau && ix <= idx_thr) out[toff++] = ix;
    });
  }
  for (int i = kk + tid; i < topk; i += kSelectThreads) out[i] = -1;
}

}  // namespace idx
