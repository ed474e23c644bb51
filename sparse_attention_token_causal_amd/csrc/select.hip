// Launchers of the per-row top-k select (select_row.hpp).
#include "select_row.hpp"

#include <algorithm>

namespace idx {

// The 1024-thread streaming variant (rows longer than any register tile)
// is held to 64 VGPRs so that two rows run per CU: one row's loads in
// flight do not cover the memory latency by themselves.
template <int NT, int KPT>
__global__ __launch_bounds__(NT, NT == 256 ? 4 : (KPT == 0 ? 8 : 1)) void select_kernel(SelectArgs a) {
  __shared__ SelectShared sh;
  select_row<NT, KPT>(a, blockIdx.x, sh);
}

template <int NT, int KPT>
static hipError_t launch_kpt(const SelectArgs& a, int rows, hipStream_t st) {
  hipLaunchKernelGGL((select_kernel<NT, KPT>), dim3(rows), dim3(NT), 0, st, a);
  return hipGetLastError();
}

// ---- rows with a scan record: one wave per row ----
//
// A filtered candidate list (dense scan) or a gathered row (Refine re-score)
// whose scan left a record with a boundary bin (or the note that the row
// holds fewer than topk candidates) is selected in one pass by one wave:
// every candidate above the boundary bin wins (the record says how many
// there are), the boundary bin's candidates (at most kFiltBoundaryMax) are
// collected in LDS and ranked exactly by (score descending, key ascending),
// the rest of the row is padded with -1.  Excluded entries (-inf, gathered
// rows only) are in no bin.  Per 64 columns the wave's winners are written
// to consecutive slots (ballot and mbcnt), so the stores are coalesced, and
// the next batch of the row is loaded while the current one is classified.
// No barrier is involved, so many rows are in flight per CU.  Returns false
// (nothing written) for a row without a usable record.
__device__ __forceinline__ bool onepass_row_wave(const SelectArgs& a, long long blk, uint32_t* lkey,
                                                 int* lidx) {
  const int l = lane_id();
  const int* fi = a.finfo + kFiltInfoStride * blk;
  const int bstar = fi[kFiltInfoBoundary];
  if (bstar == -1) return false;
  const long long frow = a.row0 + blk;
  const int b = (int)(frow / a.n_rows), r = (int)(frow % a.n_rows);
  const float* row = a.scores + blk * a.ld;
  int* out = a.out + frow * (long long)a.topk;
  const int* crow;
  if (a.mode == kModeGather) {
    const int n_g = (a.n_q + a.group - 1) / a.group;
    crow = a.cand + ((long long)b * n_g + r / a.group) * a.n_cols;
  } else {
    crow = a.lidx + blk * a.ld;
  }
  const int n = min(fi[kFiltInfoCount], a.n_cols), base = fi[kFiltInfoBase];
  const bool all = bstar == -2;  // fewer than topk candidates: all of them
  const int above = all ? n : fi[kFiltInfoAbove];
  constexpr int E = 16;  // columns per lane per batch
  // The boundary bin as a float interval [f_lo, f_hi): a key lies above the
  // bin exactly when its value is >= f_hi, in it when it is >= f_lo and
  // below f_hi (order keys are monotone in the value and map -0 to +0, and
  // the bin edges, multiples of 2^15, clamped to the keys of -FLT_MAX and
  // +inf, are keys of floats).  The edge bins also hold the keys clamped
  // into them: below the window for bin 0 (f_lo = -FLT_MAX), above it for
  // the last bin (f_hi NaN: no value compares >= it).  Excluded (-inf)
  // entries lie below both.  With fewer than topk candidates every other
  // entry lies above f_hi.
  float f_lo, f_hi;
  if (all) {
    f_hi = -__FLT_MAX__;
    f_lo = __builtin_huge_valf();
  } else {
    auto edge = [](long long kb) -> float {
      return key_to_float((uint32_t)min(max(kb, 0x00800000LL), 0xFF800000LL));
    };
    const long long kb = (long long)(bstar + base) * 32768LL;
    f_lo = bstar == 0 ? -__FLT_MAX__ : edge(kb);
    f_hi = bstar == kFiltBins - 1 ? __builtin_nanf("") : edge(kb + 32768LL);
  }
  // (32-bit byte offsets from the wave's row bases; in a row's last batch
  // the columns past its end read its last column and count as excluded)
  auto load = [&](int c0, float* vv, int* xx) {
    const bool whole = c0 + E * kWave <= n;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      int c = c0 + j * kWave + l;
      if (!whole) c = max(min(c, n - 1), 0);
      const uint32_t off = (uint32_t)c * 4u;
      vv[j] = *(const float*)((const char*)row + off);
      xx[j] = *(const int*)((const char*)crow + off);
    }
  };
  int wpos = 0, lpos = 0;
  auto classify = [&](int c0, float* v, const int* x) {
    if (c0 + E * kWave > n) {
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (c0 + j * kWave + l >= n) v[j] = neg_inf();
    }
#pragma unroll
    for (int j = 0; j < E; ++j) {
      // (each ballot is of one compare)
      const bool wn = v[j] >= f_hi;
      const unsigned long long mw = __ballot(v[j] >= f_hi), mb = __ballot(v[j] >= f_lo) & ~mw;
      const int ow = __builtin_amdgcn_mbcnt_hi((uint32_t)(mw >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mw, 0));
      if (wn && wpos + ow < a.topk) *(int*)((char*)out + (uint32_t)(wpos + ow) * 4u) = x[j];
      if (mb) {
        const int ob = __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0));
        if (((mb >> l) & 1ull) && lpos + ob < kFiltBoundaryMax) {
          lkey[lpos + ob] = order_key(v[j]);
          lidx[lpos + ob] = x[j];
        }
        lpos += __popcll(mb);
      }
      wpos += __popcll(mw);
    }
  };
  // the next batch's loads are issued before this batch is classified
  if (n > 0) {
    float v[E];
    int x[E];
    load(0, v, x);
    for (int c0 = 0; c0 < n; c0 += E * kWave) {
      float vn[E];
      int xn[E];
      const bool more = c0 + E * kWave < n;
      if (more) load(c0 + E * kWave, vn, xn);
      classify(c0, v, x);
      if (more) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
          v[j] = vn[j];
          x[j] = xn[j];
        }
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  const int m = min(lpos, kFiltBoundaryMax), need = all ? 0 : a.topk - above;
  if (need > 0) {
    for (int e = l; e < m; e += kWave) {
      const uint32_t ke = lkey[e];
      const int ie = lidx[e];
      int rank = 0;
      for (int f = 0; f < m; ++f) {
        const uint32_t kf = lkey[f];
        rank += (kf > ke || (kf == ke && lidx[f] < ie)) ? 1 : 0;
      }
      if (rank < need) out[above + rank] = ie;
    }
  }
  const int filled = min(a.topk, all ? n : above + min(need, m));
  for (int i = filled + l; i < a.topk; i += kWave) out[i] = -1;
  return true;
}

// Four rows per 256-thread workgroup, one per wave; rows without a usable
// record then run the general select (rows streamed from global memory),
// one after another with the whole workgroup.
__global__ __launch_bounds__(256, 5) void onepass_select_kernel(SelectArgs a, long long n_launch_rows) {
  __shared__ SelectShared sh;
  static_assert(4 * kFiltBoundaryMax <= kListCap, "per-wave boundary lists in the shared list");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const long long blk = (long long)blockIdx.x * 4 + wave;
  const bool done = blk >= n_launch_rows ||
                    onepass_row_wave(a, blk, sh.lkey + wave * kFiltBoundaryMax, sh.lidx + wave * kFiltBoundaryMax);
  if (lane_id() == 0) sh.wscan[wave] = done ? 0 : 1;
  __syncthreads();
  int pending = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) pending |= sh.wscan[w] << w;
  __syncthreads();
  for (int w = 0; w < 4; ++w) {
    if ((pending >> w) & 1) {
      select_row<256, 0>(a, (unsigned)(blockIdx.x * 4 + w), sh);
      __syncthreads();
    }
  }
}

static hipError_t launch_onepass(const SelectArgs& a, int rows, hipStream_t st) {
  hipLaunchKernelGGL(onepass_select_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, a, (long long)rows);
  return hipGetLastError();
}

// Smallest variant that holds a row of n keys in registers; up to 8192 keys
// 256-thread workgroups (more rows in flight per CU than wider ones), unless
// the launch has too few rows to occupy the chip (fewer than two per CU:
// decode-sized problems), where a row's chain of phases is the whole time
// and 1024 threads per row shorten it (with no more keys per thread than the
// row needs: each phase walks every register slot).
static hipError_t launch_by_length(const SelectArgs& a, int rows, int n, hipStream_t st) {
  if (rows < 512 && n > 256 * 8 && n <= 1024 * 8) return launch_kpt<1024, 8>(a, rows, st);
  if (rows < 512 && n > 256 * 8 && n <= 1024 * 16) return launch_kpt<1024, 16>(a, rows, st);
  if (n <= 256 * 8) return launch_kpt<256, 8>(a, rows, st);
  if (n <= 256 * 32) return launch_kpt<256, 32>(a, rows, st);
  if (n <= 1024 * 16) return launch_kpt<1024, 16>(a, rows, st);
  if (n <= 1024 * 32) return launch_kpt<1024, 32>(a, rows, st);
  return launch_kpt<1024, 0>(a, rows, st);
}

// Rows of a dense or proxy launch grow in length with the row index within a
// sequence; such launches are split into length classes so that each class
// runs the smallest variant that holds its rows.
hipError_t launch_select(const SelectArgs& a, int n_launch_rows, hipStream_t st) {
  // candidate lists (up to a few k (1 + ln(n / k)) entries) are held 32 keys
  // per thread by 256-thread workgroups, more rows in flight per CU than
  // with 512 threads; a longer list streams inside the kernel
  if (n_launch_rows <= 0) return hipSuccess;
  // rows with their scan's records (filtered lists, gathered rows): one wave per row
  if ((a.mode == kModeList || a.mode == kModeGather) && a.finfo) return launch_onepass(a, n_launch_rows, st);
  if (a.mode == kModeList) return launch_kpt<256, 32>(a, n_launch_rows, st);
  if (a.mode == kModeGather || n_launch_rows <= 0) return launch_by_length(a, n_launch_rows, a.n_cols, st);
  const int classes[4] = {256 * 8, 256 * 32, 1024 * 16, 1024 * 32};
  long long r = 0;
  while (r < n_launch_rows) {
    // the length of launch row r, and the longest run of rows in its class
    auto len_of = [&](long long i) {
      const long long fr = a.row0 + i;
      const int rr = (int)(fr % a.n_rows);
      const int lim = mode_limit(a.mode, a.q_pos0, a.n_q, a.group, a.block, rr);
      return std::min(lim + 1, a.n_cols);
    };
    int cls = 4;
    for (int c = 0; c < 4; ++c)
      if (len_of(r) <= classes[c]) { cls = c; break; }
    long long e = r + 1;
    while (e < n_launch_rows) {
      const int l = len_of(e);
      int ce = 4;
      for (int c = 0; c < 4; ++c)
        if (l <= classes[c]) { ce = c; break; }
      if (ce != cls) break;
      ++e;
    }
    SelectArgs sub = a;
    sub.scores = a.scores + r * a.ld;
    sub.row0 = a.row0 + r;
    const int n = cls < 4 ? classes[cls] : a.n_cols;
    hipError_t err = launch_by_length(sub, (int)(e - r), n < a.n_cols ? n : a.n_cols, st);
    if (err != hipSuccess) return err;
    r = e;
  }
  return hipSuccess;
}

// ---- top-k of the split-key scan's rows ----
//
// The compaction leaves, per row, a segmented list of every score in or
// above the row's threshold bin (bin = order key >> kSplitShift) and that
// bin.  As long as at most `need` entries lie above the bin (the usual case:
// the summed histogram only undercounts far below the row's top), all of
// them win and only the bin's own entries are ranked, for the remaining
// slots: one 2048-bin histogram of their next 11 key bits finds the sub-bin
// of the last winner, the entries above it win, and that sub-bin's entries
// are ranked exactly by (key descending, index ascending).  One pass over the
// segments (NT / n_segs threads per segment) classifies the list into LDS and
// builds that histogram; a row with more than `need` entries above the bin,
// more than kSplitBdCap in it, or more than kSplitRankCap in the last
// winner's sub-bin (runs of near-equal scores) runs the general select over
// its whole list instead.
constexpr int kSplitSelThreads = 1024;
constexpr int kSplitBdCap = 8192;
constexpr int kSplitRankCap = 256;
constexpr int kSplitSubShift = kSplitShift - 11;  // the next 11 key bits

static size_t split_select_lds(int topk) {
  return 4 * (size_t)topk + 8 * kSplitBdCap + 4 * kBins + 8 * kSplitRankCap + 4 * (kMaxSegs + 1) + 128;
}

// Slots of this lane's entries among a counter pair's reservations: `na`
// and `nb` entries of two kinds (each at most 255 per lane); one 64-bit LDS
// atomic per wave (low word: kind a, high word: kind b).  Returns the first
// slot of each kind.  Every lane of the wave must be active.
__device__ __forceinline__ void wave_reserve2(unsigned long long* counter, int na, int nb, int* pa, int* pb) {
  const int x = na | (nb << 16);
  const int incl = wave_incl_scan(x);
  const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
  unsigned long long base = 0;
  if (lane_id() == kWave - 1)
    base = atomicAdd(counter, (unsigned long long)(tot & 0xFFFF) | ((unsigned long long)(tot >> 16) << 32));
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)base, kWave - 1);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(base >> 32), kWave - 1);
  const int ex = incl - x;
  *pa = (int)lo + (ex & 0xFFFF);
  *pb = (int)hi + (ex >> 16);
}

// Exclusive prefix sum over the block (DPP within waves; wsum: one int of
// LDS per wave), with the total.
template <int NT>
__device__ __forceinline__ int block_excl_scan_dpp(int v, int* total, int* wsum) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane_id() == kWave - 1) wsum[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = wsum[i];
    before += i < w ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

__global__ __launch_bounds__(kSplitSelThreads) void split_select_kernel(SelectArgs a, const int* thr_rows,
                                                                        int lean) {
  constexpr int NT = kSplitSelThreads;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const unsigned row = blockIdx.x;
  const int tid = threadIdx.x;
  const int len =
      min(mode_limit(a.mode, a.q_pos0, a.n_q, a.group, a.block, (int)(row % a.n_rows)) + 1, a.n_cols);
  const int need = max(min(a.topk, len), 0);
  int* out = a.out + (size_t)row * a.topk;
  const float* lval = a.scores + (size_t)row * a.ld;
  const int* lkix = a.lidx + (size_t)row * a.ld;
  const int ns = a.n_segs;
  if (lean) {
    int* c_idx = (int*)lds;                                   // [topk] indices above the bin
    uint32_t* b_key = (uint32_t*)(lds + 4 * (size_t)a.topk);  // [kSplitBdCap] the bin's keys
    int* b_idx = (int*)(b_key + kSplitBdCap);                 // ... and their indices
    uint32_t* hist = (uint32_t*)(b_idx + kSplitBdCap);        // [kBins]
    uint32_t* r_key = hist + kBins;                           // [kSplitRankCap] the last sub-bin
    int* r_idx = (int*)(r_key + kSplitRankCap);
    int* soff = r_idx + kSplitRankCap;                        // [kMaxSegs + 1] segment counts
    // ctl: [0, 2) the classification's counter pair, [2, 4) the ranking's,
    // [4] the largest segment, [5] the sub-bin, [6] entries above it,
    // [8, 24) wave sums
    int* ctl = soff + kMaxSegs + 1;
    unsigned long long* cnt2 = (unsigned long long*)(((uintptr_t)ctl + 7) & ~(uintptr_t)7);
    ctl = (int*)cnt2;
    const uint32_t thr = (uint32_t)thr_rows[row];
    if (tid < 8) ctl[tid] = 0;
    for (int i = tid; i < kBins; i += NT) hist[i] = 0u;
    const int cnt = tid < ns ? a.seg_counts[(size_t)row * ns + tid] : 0;
    if (tid < ns) soff[tid] = cnt;
    __syncthreads();
    if (tid < kWave) {  // the largest segment count
      int m = 0;
      for (int i = tid; i < ns; i += kWave) m = max(m, soff[i]);
      m = (int)wave_max_u32((uint32_t)m);
      if (tid == 0) ctl[4] = m;
    }
    __syncthreads();
    // NT / ns threads per segment, 8 entries each per batch (every load of a
    // batch in flight at once)
    const int tps = NT / ns, s = tid / tps, j0 = tid - s * tps;
    const int cs = s < ns ? soff[s] : 0;
    const int mx = ctl[4];
    for (int i0 = 0; i0 < mx; i0 += 8 * tps) {
      float v[8];
      int x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int jj = i0 + j0 + j * tps;
        const size_t src = (size_t)(s < ns ? s : 0) * a.seg_len + (jj < cs ? jj : 0);
        v[j] = lval[src];
        x[j] = lkix[src];
      }
      uint32_t up = 0, in = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = i0 + j0 + j * tps < cs;
        in |= (uint32_t)ok << j;
        up |= (uint32_t)(ok && (order_key(v[j]) >> kSplitShift) > thr) << j;
      }
      const uint32_t bn = in & ~up;
      int pu, pb;
      wave_reserve2(cnt2, __builtin_popcount(up), __builtin_popcount(bn), &pu, &pb);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((up >> j) & 1u) {
          if (pu < a.topk) c_idx[pu] = x[j];
          ++pu;
        }
        if ((bn >> j) & 1u) {
          const uint32_t k = order_key(v[j]);
          atomicAdd(&hist[(k >> kSplitSubShift) & (kBins - 1)], 1u);  // the next 11 key bits
          if (pb < kSplitBdCap) {
            b_key[pb] = k;
            b_idx[pb] = x[j];
          }
          ++pb;
        }
      }
    }
    __syncthreads();
    const int above = ctl[0], nb = ctl[1], want = need - above;
    bool general = above > need || nb > kSplitBdCap || want > nb;
    if (!general && want > 0 && want < nb) {
      // thread t holds the bins from kBins - 1 - BPT t downwards
      constexpr int BPT = kBins / NT;
      int c8[BPT], sum = 0;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        c8[j] = (int)hist[kBins - 1 - (BPT * tid + j)];
        sum += c8[j];
      }
      int t8;
      int before = block_excl_scan_dpp<NT>(sum, &t8, ctl + 8);
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        if (before < want && want <= before + c8[j]) {
          ctl[5] = kBins - 1 - (BPT * tid + j);
          ctl[6] = before;
        }
        before += c8[j];
      }
      __syncthreads();
      general = (int)hist[ctl[5]] > kSplitRankCap;
    }
    if (!general) {
      for (int i = tid; i < above; i += NT) out[i] = c_idx[i];
      if (want == nb) {
        for (int i = tid; i < nb; i += NT) out[above + i] = b_idx[i];
      } else if (want > 0) {
        const uint32_t bs = (uint32_t)ctl[5];
        const int hi_n = ctl[6];  // the bin's entries above sub-bin bs: all win
        for (int i0 = 0; i0 < nb; i0 += NT) {
          const int i = i0 + tid;
          const uint32_t k = i < nb ? b_key[i] : 0u;
          const uint32_t sb = (k >> kSplitSubShift) & (kBins - 1);
          const bool hi = i < nb && sb > bs, eq = i < nb && sb == bs;
          int pu, pe;
          wave_reserve2(cnt2 + 1, hi ? 1 : 0, eq ? 1 : 0, &pu, &pe);
          if (hi) out[above + pu] = b_idx[i];
          if (eq) {
            r_key[pe] = k;
            r_idx[pe] = b_idx[i];
          }
        }
        __syncthreads();
        const int m = (int)(uint32_t)(cnt2[1] >> 32), last = want - hi_n;
        for (int e = tid; e < m; e += NT) {
          const uint32_t ke = r_key[e];
          const int ie = r_idx[e];
          int rank = 0;
          for (int f = 0; f < m; ++f) {
            const uint32_t kf = r_key[f];
            rank += (kf > ke || (kf == ke && r_idx[f] < ie)) ? 1 : 0;
          }
          if (rank < last) out[above + hi_n + rank] = ie;
        }
      }
      for (int i = need + tid; i < a.topk; i += NT) out[i] = -1;
      return;
    }
    __syncthreads();  // the general select reuses the LDS
  }
  SelectArgs g = a;
  g.row0 = 0;
  g.n_rows = 1;
  g.mode = kModeList;
  g.finfo = nullptr;
  g.scores = lval;
  g.lidx = lkix;
  g.seg_counts = a.seg_counts + (size_t)row * ns;
  g.gval = a.gval + (size_t)row * a.ld;
  g.gidx = a.gidx + (size_t)row * a.ld;
  g.out = out;
  select_row<kSplitSelThreads, 16>(g, 0u, *(SelectShared*)lds);
}

hipError_t launch_split_select(const SelectArgs& a, const int* thr, int rows, hipStream_t st) {
  if (a.n_segs < 1 || a.n_segs > kMaxSegs) return hipErrorInvalidValue;
  static bool attr_set = false;  // allow more than 64 KiB of LDS
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)split_select_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kScoreLdsMax);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t lean = split_select_lds(a.topk);
  const bool fits = lean <= kScoreLdsMax;
  const size_t lds = std::max(fits ? lean : 0, sizeof(SelectShared));
  hipLaunchKernelGGL(split_select_kernel, dim3(rows), dim3(kSplitSelThreads), lds, st, a, thr, fits ? 1 : 0);
  return hipGetLastError();
}

__global__ void fill_kernel(float* p, size_t n, float v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill(float* p, size_t n, float v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace idx
