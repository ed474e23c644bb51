// Causal indexer score kernel for gfx950.
//
// Computes I[t, s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]) for a block of
// rows (queries, or PIVOT proxies) against a range of key columns.  The key
// columns are either the positions 0..n_k-1 of the sequence (dense scan and
// proxy scan) or a per-group candidate list (PIVOT-Refine re-score, keys
// gathered by index).  Sources: "PIVOT: Efficient Query-Group Indexing for
// Token-Level Sparse Attention", Abstract (score every preceding token; one
// shared proxy scan; re-score the candidates per query); "ADIndex ...",
// "Why the Indexer Becomes the Bottleneck" (whole causal prefix per query).
//
// Contraction on MFMA: rows = (query, head) pairs, columns = keys, inner
// dimension = the head dimension d.  A wave owns 64 rows (two 32-row MFMA
// blocks = 64/H queries) with its q fragments resident in registers, and 64
// key columns per step (two 32-column blocks).  The 32x32 MFMA result layout
// puts 16 rows of one column in each lane (row = 8*(v/4) + 4*(lane/32) + v%4,
// column = lane%32), so the head reduction is an in-lane weighted sum plus
// one exchange with lane^32.  The epilogue (ReLU, x w, sum over heads,
// per-token FP8 scales, causal mask) runs on those registers; only the
// per-(query, key) score leaves the wave.
//
// Key tiles are staged in LDS once per workgroup and read by every wave;
// rows are padded by 16 bytes so that the 16-byte fragment reads of 16
// consecutive lanes hit distinct banks.  FP8 keys scanned with bfloat16
// queries are widened to bfloat16 while staged (exact).
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace idx {

template <int QF, int KF>
struct MfmaTraits;

// float32 x float32: v_mfma_f32_32x32x2_f32, one element of k per lane half.
template <>
struct MfmaTraits<F32, F32> {
  static constexpr int KSTEP = 2, KE = 4, GE = 4;
  typedef float frag;
  __device__ static frag load_a(const char* rowp, int ks, int half) {
    return *(const float*)(rowp + (ks * 2 + half) * 4);
  }
  __device__ static frag load_b(const char* ldsrow, int ks, int half) {
    return *(const float*)(ldsrow + (ks * 2 + half) * 4);
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// bfloat16 x bfloat16: v_mfma_f32_32x32x16_bf16, 8 consecutive k per lane half.
struct MfmaBf16 {
  static constexpr int KSTEP = 16, KE = 2;
  typedef bf16x8 frag;
  __device__ static frag load_a(const char* rowp, int ks, int half) {
    return *(const bf16x8*)(rowp + (ks * 16 + 8 * half) * 2);
  }
  __device__ static frag load_b(const char* ldsrow, int ks, int half) {
    return *(const bf16x8*)(ldsrow + (ks * 16 + 8 * half) * 2);
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct MfmaTraits<BF16, BF16> : MfmaBf16 {
  static constexpr int GE = 2;
};
template <>
struct MfmaTraits<BF16, FP8> : MfmaBf16 {
  static constexpr int GE = 1;  // staged from FP8, widened to bfloat16 in LDS
};

// FP8 x FP8: v_mfma_f32_32x32x64_f8f6f4 (both operands E4M3), 32 consecutive k per lane half.
template <>
struct MfmaTraits<FP8, FP8> {
  static constexpr int KSTEP = 64, KE = 1, GE = 1;
  typedef i32x8 frag;
  __device__ static frag load_a(const char* rowp, int ks, int half) {
    const i32x4* p = (const i32x4*)(rowp + ks * 64 + 32 * half);
    i32x4 x = p[0], y = p[1];
    frag f = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return f;
  }
  __device__ static frag load_b(const char* ldsrow, int ks, int half) {
    const i32x4* p = (const i32x4*)(ldsrow + ks * 64 + 32 * half);
    i32x4 x = p[0], y = p[1];
    frag f = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return f;
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

__device__ __forceinline__ int row_limit(const ScoreArgs& a, int r) {
  return mode_limit(a.mode, a.q_pos0, a.n_q, a.group, a.block, r);
}

// Scheduling groups for the instruction scheduler (gfx9 sched_group_barrier masks).
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;

// GATHER: columns are the group's candidate list (PIVOT-Refine); otherwise the
// columns are key positions (dense scan, proxy scan).
// Filtering: bins of the running per-row histogram (256 per octave of the
// score, a window of 8 octaves placed from the first tile's largest score).

// FILTER: 0 full score rows; 1 the filtering scan (candidate lists); 2 the
// rescan of the row blocks whose lists overflowed; 3 full score rows of
// gathered columns plus each row's record of its exact boundary bin (see
// ScoreArgs::filter).
template <int QF, int KF, int H, int D, int RW, bool GATHER, int NWV, int FILTER>
__global__ __launch_bounds__(NWV * 64) void score_kernel(ScoreArgs a) {
  constexpr int kScoreThreads = NWV * 64;  // threads of this workgroup
  typedef MfmaTraits<QF, KF> M;
  constexpr int NKS = D / M::KSTEP;
  constexpr int ROWB = D * M::KE + 16;
  constexpr int QW = 64 / H;                  // queries per wave
  constexpr int NW = NWV;                     // waves per workgroup
  constexpr int KW = NW / RW, TW = KW * 64;   // key-waves, tile width (columns)
  constexpr bool WIDEN = (KF == FP8 && QF == BF16);
  constexpr int CPC = D * M::GE / 16;         // 16-byte global chunks per key row
  constexpr int NCH = (TW * CPC + kScoreThreads - 1) / kScoreThreads;  // chunks per thread per tile
  constexpr int TILE_BYTES = TW * ROWB + TW * 8;
  // per-column data (key index, key scale) is only needed for gathered
  // columns or FP8 keys; dense scans of BF16/F32 keys use the position itself
  constexpr bool COLINFO = GATHER || KF == FP8;
  static_assert(FILTER == 0 || (QW == 1 && (GATHER ? FILTER == 3 : FILTER != 3)),
                "filtering: dense scans, records: gathered columns; one query per wave");

  // two tile buffers: [TW][ROWB] key rows, then TW column keys and TW scales
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int wave = threadIdx.x / kWave, l = lane_id(), half = l >> 5, l32 = l & 31;
  const int rw = wave % RW, kw = wave / RW;
  constexpr int BQ = RW * QW;

  // Rescan state of this wave's row (wave-uniform), kept in registers across
  // the levels of one row block: the row is pending while its list cannot
  // hold every key at or above the boundary interval [r_lo, r_hi]; r_A keys
  // lie above it (all of them win) and the (topk - r_A)-th largest key of
  // the interval is the row's last winner.
  bool r_act = false;
  uint32_t r_lo = 0u, r_hi = 0u;
  int r_A = 0;

  // Workgroup-wide "any" of a wave-uniform flag, through one int per wave
  // after the filter histograms (the leading barrier retires the previous
  // call's reads).
  auto wg_any = [&](bool p) -> bool {
    int* flags = (int*)(smem + 2 * TILE_BYTES + NW * kFiltBins * 4);
    __syncthreads();
    if (l == 0) flags[wave] = p ? 1 : 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) any |= flags[i];
    return any != 0;
  };

  // The scan of one row block; the rescan (FILTER == 2) returns whether a
  // row of the block is still pending after this level.
  auto run = [&](const int bid, const int level) -> bool {
  // ---- which rows this workgroup owns (longest prefixes first) ----
  int b, r_begin, r_end, g = 0;
  if (!GATHER) {
    const int bps = (a.n_rows + BQ - 1) / BQ;
    b = bid / bps;
    r_begin = (bid % bps) * BQ;
    r_end = min(r_begin + BQ, a.n_rows);
  } else {
    const int n_g = (a.n_q + a.group - 1) / a.group;
    const int bpg = (a.group + BQ - 1) / BQ;
    b = bid / (n_g * bpg);
    g = (bid / bpg) % n_g;
    const int gs = g * a.group, ge = min(gs + a.group, a.n_q);
    r_begin = gs + (bid % bpg) * BQ;
    r_end = min(r_begin + BQ, ge);
    if (r_begin >= r_end) return false;
  }
  const int c_begin = (int)blockIdx.y * a.kc;
  int c_end = min(c_begin + a.kc, a.n_cols);
  if (!GATHER) c_end = min(c_end, row_limit(a, r_end - 1) + 1);
  if (c_begin >= c_end) return false;
  const int t_first = r_begin + rw * QW;

  // ---- the row's list, record and (rescan) state ----
  long long crow = 0;
  int* info = nullptr;
  if constexpr (FILTER != 0) {
    crow = (long long)b * a.n_rows + t_first - a.row0;
    if (t_first < r_end) info = a.ccount + kFiltInfoStride * crow;
  }
  bool r_tie = false;
  int r_need = 0, r_shift = 0;
  if constexpr (FILTER == 2) {
    if (level == 0) {
      r_act = false;
      if (info) {
        r_act = __builtin_amdgcn_readfirstlane(info[kFiltInfoStatus]) != 0;
        r_lo = (uint32_t)__builtin_amdgcn_readfirstlane(info[kFiltInfoLo]);
        r_hi = (uint32_t)__builtin_amdgcn_readfirstlane(info[kFiltInfoHi]);
        r_A = __builtin_amdgcn_readfirstlane(info[kFiltInfoA]);
      }
    }
    // nothing pending in this block: the workgroup skips it (also the
    // barrier that retires the previous block's LDS reads)
    if (!wg_any(r_act)) return false;
    r_tie = r_lo == r_hi;
    r_need = a.topk - r_A;
    // bins of the class histogram: 2048 over [r_lo, r_hi]
    while (((r_hi - r_lo) >> r_shift) >= (uint32_t)kFiltBins) ++r_shift;
  }

  // ---- resident q fragments and head weights of this wave's 64 rows ----
  typename M::frag afrag[2][NKS];
  float wreg[2][16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int i = 32 * rb + l32;  // A-operand row of this lane
    const int t = t_first + i / H, h = i % H;
    const bool ok = t < r_end;
    const char* rowp = (const char*)a.q + (((size_t)b * a.n_rows + (ok ? t : r_begin)) * H + h) * (size_t)D * (QF == F32 ? 4 : (QF == BF16 ? 2 : 1));
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      typename M::frag f = M::load_a(rowp, ks, half);
      if (!ok) f = typename M::frag{};
      afrag[rb][ks] = f;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ri = 32 * rb + 8 * (v / 4) + 4 * half + (v % 4);  // C-result row of register v
      const int tt = t_first + ri / H, hh = ri % H;
      float wv = 0.f;
      if (tt < r_end) {
        const size_t fr = (size_t)b * a.n_rows + tt;
        wv = a.w[fr * H + hh];
        if (QF == FP8) wv *= a.q_scale[fr];
      }
      wreg[rb][v] = wv;
    }
  }

  // ---- filtering state (one query per wave; wave-uniform) ----
  // The scan counts every candidate (f_cnt) and stores the first cld of
  // them; the rescan counts the interval's keys in `hist` (bins of
  // 2^r_shift above r_lo) and, on a tied interval, c_cnt of its keys so far.
  // (after the candidate indices when the columns are gathered)
  // The records of gathered rows count at most kCandLdsMax columns per row,
  // so their bins are 16-bit counters, two per word (the filtering scan and
  // the rescan count up to a whole prefix: one word per bin).
  constexpr int HW = FILTER == 3 ? kFiltBins / 2 : kFiltBins;  // histogram words per wave
  static_assert(kCandLdsMax < 65536, "a record's bin counts fit 16 bits");
  uint32_t* hist = (uint32_t*)(smem + 2 * TILE_BYTES + (GATHER ? (a.kc * 4 + 15) / 16 * 16 : 0)) + wave * HW;
  auto hist_count = [&](int bin) -> int {
    return FILTER == 3 ? (int)((hist[bin >> 1] >> (16 * (bin & 1))) & 0xFFFFu) : (int)hist[bin];
  };
  int f_base = 0, f_theta = 0, f_above = 0, f_cnt = 0, c_cnt = 0;
  float f_lo = neg_inf();  // lower edge of bin f_theta (-inf while f_theta == 0)
  bool f_based = false;
  float* f_val = nullptr;
  int* f_idx = nullptr;
  if constexpr (FILTER != 0) {
    for (int i = l; i < HW; i += kWave) hist[i] = 0;
    if constexpr (FILTER != 3) {
      f_val = a.cval + crow * a.cld;
      f_idx = a.cidx + crow * a.cld;
    }
  }

  // Gathered columns: the workgroup's candidate key indices are copied to
  // LDS once (after the tile buffers), so staging a key tile reads them from
  // LDS instead of issuing global loads that the key-row loads depend on.
  int* s_cand = (int*)(smem + 2 * TILE_BYTES);
  if constexpr (GATHER) {
    const int* cand_row = a.cand + ((size_t)b * ((a.n_q + a.group - 1) / a.group) + g) * a.n_cols;
    for (int i = threadIdx.x; i < c_end - c_begin; i += kScoreThreads) s_cand[i] = cand_row[c_begin + i];
    __syncthreads();
  }
  const char* kseq = (const char*)a.k + (size_t)b * a.n_k * D * M::GE;

  // ---- staging of one key tile: global -> registers -> LDS (double buffered) ----
  // Loads are unconditional: a column past the range or an empty candidate
  // slot reads a valid key row (it is masked in the epilogue), so the loads
  // of a tile are all in flight together while the current tile computes.
  // The FP8 key scales travel with the key rows (loaded with them, two tiles
  // ahead): a scale loaded only when the tile is stored would expose a full
  // memory latency before every tile's barrier.
  i32x4 stage_buf[2][NCH];
  int stage_keys[2][NCH];
  float stage_scl[2][NCH];
  // Gathered columns: the key indices of a tile are read from LDS one tile
  // before its loads are issued (stage_index), so that the loads do not wait
  // for an LDS round trip.
  auto stage_index = [&](auto set_c, int c0) {
    if constexpr (GATHER) {
      constexpr int SET = decltype(set_c)::value;
#pragma unroll
      for (int u = 0; u < NCH; ++u) {
        const int i = min((int)threadIdx.x + u * kScoreThreads, TW * CPC - 1);
        const int j = i / CPC;
        int s = s_cand[min(c0 + j, c_end - 1) - c_begin];
        if (c0 + j >= c_end || s >= a.n_k) s = -1;
        stage_keys[SET][u] = s;
      }
    }
  };
  auto stage_load = [&](auto set_c, int c0) {
    constexpr int SET = decltype(set_c)::value;
    i32x4* stage = stage_buf[SET];
    int* stage_key = stage_keys[SET];
    float* stage_sc = stage_scl[SET];
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int i = min((int)threadIdx.x + u * kScoreThreads, TW * CPC - 1);
      const int j = i / CPC, c = i % CPC;
      int srow;
      if (GATHER) {
        srow = max(stage_key[u], 0);
      } else {
        const int col = min(c0 + j, c_end - 1);
        stage_key[u] = c0 + j < c_end ? col : -1;
        srow = col;
      }
      stage[u] = *(const i32x4*)(kseq + ((size_t)srow * D * M::GE) + c * 16);
      if constexpr (KF == FP8) stage_sc[u] = a.k_scale[(size_t)b * a.n_k + srow];
    }
  };
  auto stage_store = [&](auto set_c, int buf) {
    constexpr int SET = decltype(set_c)::value;
    const i32x4* stage = stage_buf[SET];
    const int* stage_key = stage_keys[SET];
    const float* stage_sc = stage_scl[SET];
    char* kt = smem + buf * TILE_BYTES;
    int* ck = (int*)(kt + TW * ROWB);
    float* cs = (float*)(ck + TW);
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int i = threadIdx.x + u * kScoreThreads;
      if (NCH * kScoreThreads == TW * CPC || i < TW * CPC) {
        const int j = i / CPC, c = i % CPC;
        const i32x4 v = stage[u];
        if (WIDEN) {
          uint32_t o[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) fp8x4_to_bf16x4((uint32_t)v[e], o[2 * e], o[2 * e + 1]);
          i32x4* dst = (i32x4*)(kt + j * ROWB + c * 32);
          dst[0] = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
          dst[1] = i32x4{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
        } else {
          *(i32x4*)(kt + j * ROWB + c * 16) = v;
        }
        if (COLINFO && c == 0) {
          const int s = stage_key[u];
          ck[j] = s;
          cs[j] = (s >= 0 && KF == FP8) ? stage_sc[u] : 1.f;
        }
      }
    }
  };

  // ---- MFMA of one 32-column block over d, from LDS buffer `buf` ----
  // (zero before the first tile: its epilogue reads the blocks of a tile
  // that does not exist, and discards them)
  f32x16 acc[2][2] = {};
  // With few inner steps (bf16, fp8) the fragments of a block are read from
  // LDS ahead of its MFMAs: block 0's at the top of the tile, block 1's while
  // block 0 computes.  Float32 (64 steps) reads step by step.
  constexpr bool PRELOAD = NKS <= 8;
  typedef typename M::frag frag_t;
  frag_t bfA[PRELOAD ? NKS : 1], bfB[PRELOAD ? NKS : 1];
  auto load_block = [&](frag_t* bf, int buf, int cb) {
    const char* ldsrow = smem + buf * TILE_BYTES + (kw * 64 + cb * 32 + l32) * ROWB;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bf[ks] = M::load_b(ldsrow, ks, half);
  };
  auto mfma_block = [&](const frag_t* bf, int buf, int cb) {
    if constexpr (PRELOAD) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb][cb] = M::mma(afrag[rb][ks], bf[ks], ks == 0 ? f32x16{} : acc[rb][cb]);
    } else {
      const char* ldsrow = smem + buf * TILE_BYTES + (kw * 64 + cb * 32 + l32) * ROWB;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const frag_t b1 = M::load_b(ldsrow, ks, half);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb][cb] = M::mma(afrag[rb][ks], b1, ks == 0 ? f32x16{} : acc[rb][cb]);
      }
    }
  };
  constexpr int NDSR = NKS * (int)(sizeof(frag_t) / 16);  // 16-byte LDS reads per block
  // Where a tile's block 0 partial sums run: beside block 1's MFMAs when
  // those take longer than the sums (bf16: 16 MFMAs of 32 cycles per block;
  // float32), else at the top of the next tile (FP8: 4 MFMAs of 64 cycles).
  constexpr bool LATE0 = M::KSTEP <= 16;
  // one MFMA per few VALU ops, optionally with the next block's fragment reads spread in
#define IDX_INTERLEAVE(id, reads)                                                      \
  if constexpr (PRELOAD) {                                                             \
    _Pragma("unroll") for (int i_ = 0; i_ < 2 * NKS; ++i_) {                           \
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, id);                         \
      __builtin_amdgcn_sched_group_barrier(kSchedVALU, 4, id);                         \
      if ((reads) && i_ < NDSR) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, id); \
    }                                                                                  \
  }


  // ---- epilogue: ReLU, x w, sum over heads, scale, mask, store ----
  // The head sum is an in-lane weighted sum over the 16 result rows the lane
  // holds (`partial`, one 32-column block), plus the other half-wave's
  // partial.  One v_permlane32_swap of the two blocks' partials leaves lane
  // l < 32 with both halves of block 0's column l and lane l >= 32 with both
  // halves of block 1's column l - 32, so the rest of the epilogue (mask,
  // scale, store or filter) runs once per tile on 64 distinct columns:
  // lane l owns column kw*64 + l of tile c0, described by `key`/`scale`.
  auto partial = [&](int cb, float* pout) {
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      float ps[4] = {0.f, 0.f, 0.f, 0.f};  // four independent FMA chains
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if ((32 * rb + 8 * (v / 4)) / H == qi) {
            // ReLU as an integer max of the bits: negative floats (and -0)
            // are negative integers, so they become +0 (one VALU op, no
            // NaN canonicalisation)
            const float r = __int_as_float(max(__float_as_int(acc[rb][cb][v]), 0));
            ps[v & 3] = __builtin_fmaf(wreg[rb][v], r, ps[v & 3]);
          }
      pout[qi] = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
  };
  // last visible key of each of this wave's queries (-1 past the row range)
  int qlim[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) qlim[qi] = t_first + qi < r_end ? row_limit(a, t_first + qi) : -1;
  auto epilogue = [&](const float* p0, const float* p1, int c0, int key, float scale, bool live) {
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0[qi]), __float_as_uint(p1[qi]), false,
                                                       false);
      const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int t = t_first + qi;
      const int col = c0 + kw * 64 + l;
      const bool mine = live && t < r_end && col < c_end;
      const bool ok = mine && key >= 0 && key <= qlim[qi];
      const float val = ok ? (KF == FP8 ? tot * scale : tot) : neg_inf();
      if constexpr (FILTER == 0 || FILTER == 3) {
        if (mine) a.out[((size_t)b * a.n_rows + t - a.row0) * a.ld + col] = val;
        if constexpr (FILTER == 3) {
          // every eligible score in the row's histogram (bins placed from the
          // first tile as in the filtering scan)
          if (!f_based) {
            // (DPP lane moves: a chain of LDS-routed shuffles here was
            // executed on every tile, its latency exposed each time)
            const uint32_t m = wave_max_u32(ok ? order_key(val) : 0u);
            if (m != 0u) {
              f_base = (int)(m >> 15) - (kFiltBins - 512);
              f_based = true;
            }
          }
          if (ok) {
            const int bin = min(max((int)(order_key(val) >> 15) - f_base, 0), kFiltBins - 1);
            atomicAdd(&hist[bin >> 1], 1u << (16 * (bin & 1)));
          }
        }
      } else if constexpr (FILTER == 2) {
        // Rescan: keys above the interval are always stored; the interval's
        // keys are stored while they fit and counted in the class histogram,
        // or, on an exactly tied interval, only the first r_need of them in
        // key order (ties go to the lower index, and columns arrive in
        // increasing order: tile by tile, lane by lane).
        const uint32_t kv = ok ? order_key(val) : 0u;
        const bool abv = r_act && ok && kv > r_hi;
        const bool cls = r_act && ok && kv >= r_lo && kv <= r_hi;
        const unsigned long long lt = (l == 0) ? 0ull : (~0ull >> (kWave - l));
        bool wr = abv || cls;
        if (r_tie) {
          const unsigned long long cm = __ballot(cls);
          wr = abv || (cls && c_cnt + __popcll(cm & lt) < r_need);
          c_cnt += __popcll(cm);
        } else if (cls) {
          atomicAdd(&hist[(kv - r_lo) >> r_shift], 1u);
        }
        const unsigned long long pm = __ballot(wr);
        if (wr) {
          const int off = f_cnt + __popcll(pm & lt);
          if (off < a.cld) {
            f_val[off] = val;
            f_idx[off] = key;
          }
        }
        f_cnt += __popcll(pm);
      } else {
        // Running threshold: f_theta is a bin with at least topk counted
        // scores at or above it, so its lower edge f_lo bounds the row's final
        // k-th score from below and a score under it cannot be in the top-k.
        // Only passing scores are counted: bins under the threshold are never
        // consulted again.
        if (!f_based) {
          // (DPP lane moves: a chain of LDS-routed shuffles here was
          // executed on every tile, its latency exposed each time)
          const uint32_t m = wave_max_u32(ok ? order_key(val) : 0u);
          if (m != 0u) {
            f_base = (int)(m >> 15) - (kFiltBins - 512);
            f_based = true;
          }
        }
        const bool pass = ok && val >= f_lo;
        const unsigned long long pm = __ballot(pass);
        if (pm) {
          if (pass) {
            const int bin = min(max((int)(order_key(val) >> 15) - f_base, 0), kFiltBins - 1);
            atomicAdd(&hist[bin], 1u);
            const unsigned long long lt = (l == 0) ? 0ull : (~0ull >> (kWave - l));
            const int off = f_cnt + __popcll(pm & lt);
            if (off < a.cld) {  // beyond the list: counted, left to the rescan
              f_val[off] = val;
              f_idx[off] = key;
            }
          }
        }
        const int np = __popcll(pm);
        f_cnt += np;
        f_above += np;
      }
    }
  };

  // Raise the threshold bin: advance over the lowest bins at or above it while
  // at least topk counted scores remain above them.  One gather of 64 bins,
  // a wave prefix sum and a ballot move it up to 64 bins at a time.  Called
  // every eight tiles: a stale threshold only admits extra candidates, and
  // each call is a chain of dependent LDS and cross-lane steps that the
  // wave cannot overlap with its MFMAs (every four tiles cost about 3% more
  // scan time than every eight, every sixteen about the same).
  auto advance_theta = [&]() {
    for (;;) {
      const int bi = f_theta + l;
      const int h = bi < kFiltBins ? (int)hist[bi] : 0;
      const int incl = wave_incl_scan(h);
      const unsigned long long mv = __ballot(bi < kFiltBins - 1 && f_above - incl >= a.topk);
      const int J = __popcll(mv);  // a prefix of the lanes: incl is nondecreasing
      if (J == 0) break;
      f_above -= __builtin_amdgcn_readlane(incl, J - 1);
      f_theta += J;
      // smallest key of bin f_theta (bins above 0 start at (f_theta + f_base) << 15;
      // a non-positive start means every key lies at or above it)
      f_lo = (f_theta + f_base) > 0 ? key_to_float((uint32_t)(f_theta + f_base) << 15) : neg_inf();
      if (J < kWave) break;
    }
  };

  // ---- software-pipelined scan over the key tiles ----
  // While the MFMAs of one column block run, the epilogue of the other block
  // (of this tile or of the previous one) executes on the VALU; the next
  // tile's global loads are in flight meanwhile, and one barrier per tile
  // publishes the next LDS buffer.
  // Global loads run two tiles ahead of the MFMAs (two register staging sets;
  // set P holds the tiles of parity P between their load and their store).
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  stage_index(S0{}, c_begin);
  stage_load(S0{}, c_begin);
  stage_index(S1{}, c_begin + TW);
  if (c_begin + TW < c_end) stage_load(S1{}, c_begin + TW);
  stage_store(S0{}, 0);
  stage_index(S0{}, c_begin + 2 * TW);
  __syncthreads();
  int buf = 0, prev_c0 = c_begin, key_prev = -1;
  float scale_prev = 1.f;
  float p0_prev[QW], p1[QW];  // partial head sums of the previous tile's blocks
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) p0_prev[qi] = 0.f;
  const int jl = kw * 64 + l;
  auto tile = [&](auto par_c, int c0) {
    constexpr int PAR = decltype(par_c)::value;  // parity of this tile's index
    using Cur = std::integral_constant<int, PAR>;
    using Nxt = std::integral_constant<int, 1 - PAR>;
    // unconditional (addresses clamped into the range): the compiler then
    // counts these loads on every path and waits only for the older set
    // before storing it, instead of for every load in flight
    stage_load(Cur{}, c0 + 2 * TW);
    int key_cur = c0 + jl;
    float scale_cur = 1.f;
    if (COLINFO) {
      const int* ck = (const int*)(smem + buf * TILE_BYTES + TW * ROWB);
      key_cur = ck[jl];
      scale_cur = ((const float*)(ck + TW))[jl];
    }
    if constexpr (PRELOAD) load_block(bfA, buf, 0);
    // FP8: the previous tile's block 0 partials while block 0's fragments
    // arrive (consumed before block 0's MFMAs overwrite its accumulators)
    if constexpr (!LATE0) partial(0, p0_prev);
    // block 0 MFMAs || the previous tile's block 1 partials and its epilogue
    // (nothing is stored on the first tile) || block 1 fragment reads
    mfma_block(bfA, buf, 0);
    partial(1, p1);
    epilogue(p0_prev, p1, prev_c0, key_prev, scale_prev, c0 != c_begin);
    if constexpr (PRELOAD) load_block(bfB, buf, 1);
    IDX_INTERLEAVE(0, true);
    // block 1 MFMAs || (bf16, float32) this tile's block 0 partials, kept
    // here by an empty use (the compiler would sink them past the barrier
    // into the next tile's serial start)
    mfma_block(bfB, buf, 1);
    if constexpr (LATE0) {
      partial(0, p0_prev);
#pragma unroll
      for (int qi = 0; qi < QW; ++qi) __asm__ __volatile__("" ::"v"(p0_prev[qi]));
      IDX_INTERLEAVE(1, false);
    }
    if constexpr (FILTER == 1) {
      if ((((c0 - c_begin) / TW) & 7) == 7) advance_theta();
    }
    if (c0 + TW < c_end) stage_store(Nxt{}, buf ^ 1);
    stage_index(Nxt{}, c0 + 3 * TW);
    __syncthreads();
    prev_c0 = c0;
    key_prev = key_cur;
    scale_prev = scale_cur;
    buf ^= 1;
  };
  // whole pairs of tiles, then an odd last tile (a loop body without a
  // conditional second tile: the compiler's wait counts at the loop head
  // then only see the path where both staging sets were consumed)
  int c0 = c_begin;
  for (; c0 + TW < c_end; c0 += 2 * TW) {
    tile(S0{}, c0);
    tile(S1{}, c0 + TW);
  }
  if (c0 < c_end) tile(S0{}, c0);
  if constexpr (!LATE0) partial(0, p0_prev);
  partial(1, p1);
  epilogue(p0_prev, p1, prev_c0, key_prev, scale_prev, true);
  // The bin where the count from the top of `hist` reaches `need`: returns
  // it (-2 when the histogram holds fewer), with the count in bins above it
  // and in it.
  auto boundary_bin = [&](int need, int& above, int& cnt_b) -> int {
    above = 0;
    cnt_b = 0;
    for (int hi = kFiltBins; hi > 0; hi -= kWave) {
      const int h = hist_count(hi - 1 - l);  // lane j: bin hi - 1 - j (from the top)
      const int incl = wave_incl_scan(h);
      const unsigned long long m = __ballot(above + incl >= need);
      if (m) {
        const int J = __builtin_ctzll(m);
        const int hJ = __shfl(h, J, kWave), iJ = __shfl(incl, J, kWave);
        cnt_b = hJ;
        above += iJ - hJ;
        return hi - 1 - J;
      }
      above += __shfl(incl, kWave - 1, kWave);
    }
    return -2;
  };
  if constexpr (FILTER == 3) {
    // The row's exact boundary bin and the count above it, when this
    // workgroup saw every column of the row; the select then writes the bins
    // above it and ranks only that bin (the general path otherwise: a large
    // or clamped boundary bin, fewer eligible keys than topk, or columns
    // split over workgroups).
    int above, cnt_b;
    const int bstar = boundary_bin(a.topk, above, cnt_b);
    if (l == 0 && t_first < r_end) {
      const bool whole = a.kc >= a.n_cols;
      info[kFiltInfoCount] = a.n_cols;
      info[kFiltInfoBase] = f_base;
      info[kFiltInfoBoundary] =
          (whole && bstar > 0 && bstar < kFiltBins - 1 && cnt_b <= kFiltBoundaryMax) ? bstar : -1;
      info[kFiltInfoAbove] = above;
    }
  }
  if constexpr (FILTER == 1) {
    // The histogram counts every candidate in its bin, so the bin where the
    // count from the top reaches topk (and the count above it) is exact:
    // the select then only ranks that bin's candidates.  A row with more
    // candidates than its list holds is left pending for the rescan, which
    // starts from the whole key range.
    int above, cnt_b;
    const int bstar = boundary_bin(a.topk, above, cnt_b);
    const bool ovf = t_first < r_end && f_cnt > a.cld;
    if (l == 0 && t_first < r_end) {
      info[kFiltInfoCount] = f_cnt;
      info[kFiltInfoBase] = f_base;
      info[kFiltInfoBoundary] = (!ovf && (bstar == -2 || cnt_b <= kFiltBoundaryMax)) ? bstar : -1;
      info[kFiltInfoAbove] = above;
      info[kFiltInfoStatus] = ovf ? 1 : 0;
      info[kFiltInfoLo] = 1;            // every eligible order key is >= 1
      info[kFiltInfoHi] = (int)0xFFFFFFFFu;
      info[kFiltInfoA] = 0;
    }
    if (wg_any(ovf) && threadIdx.x == 0) {
      const int j = atomicAdd(a.ovf_count, 1);
      a.ovf_list[j] = bid;
    }
  }
  if constexpr (FILTER == 2) {
    bool pend = false;
    int d = 0, above = 0, cnt_b = 0;
    // narrow the interval to the bin of its r_need-th largest key (the
    // interval holds at least r_need keys: d >= 0 whenever f_cnt > cld)
    if (r_act && !r_tie && f_cnt > a.cld) d = boundary_bin(r_need, above, cnt_b);
    if (r_act) {
      if (r_tie || f_cnt <= a.cld || d < 0) {
        // every key at or above the interval is stored (on a tied interval
        // exactly topk of them): the select's general path ranks the list
        if (l == 0) {
          info[kFiltInfoCount] = min(f_cnt, (int)a.cld);
          info[kFiltInfoBoundary] = -1;
          info[kFiltInfoAbove] = 0;
          info[kFiltInfoStatus] = 0;
        }
        r_act = false;
      } else {
        r_lo += (uint32_t)d << r_shift;
        // the bin's last key, saturated at the top of the key range
        const unsigned long long top = (unsigned long long)r_lo + ((1ull << r_shift) - 1ull);
        r_hi = top < (unsigned long long)r_hi ? (uint32_t)top : r_hi;
        r_A += above;
        pend = true;
      }
    }
    return wg_any(pend);
  }
  return false;
  };  // run

  if constexpr (FILTER == 2) {
    // the overflowed row blocks of this launch's chunk, each rescanned until
    // all its rows are resolved (at most kRescanLevels levels)
    const int n_over = *a.ovf_count;
    for (int j = (int)blockIdx.x; j < n_over; j += (int)gridDim.x) {
      const int bid = a.ovf_list[j];
      for (int level = 0; level < kRescanLevels; ++level)
        if (!run(bid, level)) break;
    }
  } else {
    run(a.blk0 + (a.n_blocks - 1 - (int)blockIdx.x), 0);
  }
#undef IDX_INTERLEAVE
}

template <int QF, int KF, int H, int D, int RW, bool GATHER, int NWV, int FILTER = 0>
static hipError_t launch_mode(const ScoreArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  static bool attr_set = false;  // once per instantiation: allow more than 64 KiB of LDS
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)score_kernel<QF, KF, H, D, RW, GATHER, NWV, FILTER>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kScoreLdsMax);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((score_kernel<QF, KF, H, D, RW, GATHER, NWV, FILTER>), grid, dim3(NWV * 64), lds, st, a);
  return hipGetLastError();
}

// Workgroups of 8 waves, or of 4 row-waves (two independent workgroups per CU).
template <int QF, int KF, int H, int D, int RW>
static hipError_t launch_one(const ScoreArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  const bool g = a.mode == kModeGather;
  if constexpr (H == 64 && RW == 8) {
    if (a.filter == 1 && !g) return launch_mode<QF, KF, H, D, 8, false, 8, 1>(a, grid, lds, st);
    if (a.filter == 2 && !g) return launch_mode<QF, KF, H, D, 8, false, 8, 2>(a, grid, lds, st);
    if (a.filter == 3 && g) return launch_mode<QF, KF, H, D, 8, true, 8, 3>(a, grid, lds, st);
  }
  if (a.filter != 0) return hipErrorInvalidValue;
  if (RW == 4 && a.nw == 4)
    return g ? launch_mode<QF, KF, H, D, 4, true, 4>(a, grid, lds, st)
             : launch_mode<QF, KF, H, D, 4, false, 4>(a, grid, lds, st);
  return g ? launch_mode<QF, KF, H, D, RW, true, 8>(a, grid, lds, st)
           : launch_mode<QF, KF, H, D, RW, false, 8>(a, grid, lds, st);
}

template <int QF, int KF, int H, int D>
static hipError_t pick_rw(const ScoreArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  if (a.rw == 2) return launch_one<QF, KF, H, D, 2>(a, grid, lds, st);
  if (a.rw == 4) return launch_one<QF, KF, H, D, 4>(a, grid, lds, st);
  if (a.rw == 8) return launch_one<QF, KF, H, D, 8>(a, grid, lds, st);
  return hipErrorInvalidValue;
}

template <int QF, int KF, int H>
static hipError_t pick_d(const ScoreArgs& a, int D, dim3 grid, size_t lds, hipStream_t st) {
  if (D == 64) return pick_rw<QF, KF, H, 64>(a, grid, lds, st);
  if (D == 128) return pick_rw<QF, KF, H, 128>(a, grid, lds, st);
  return hipErrorInvalidValue;
}

template <int QF, int KF>
static hipError_t pick_h(const ScoreArgs& a, int H, int D, dim3 grid, size_t lds, hipStream_t st) {
  if (H == 16) return pick_d<QF, KF, 16>(a, D, grid, lds, st);
  if (H == 32) return pick_d<QF, KF, 32>(a, D, grid, lds, st);
  if (H == 64) return pick_d<QF, KF, 64>(a, D, grid, lds, st);
  return hipErrorInvalidValue;
}

size_t score_lds_bytes(int qf, int kf, int D, int rw, int nw, int filter, int gather_cols) {
  const int ke = (qf == F32) ? 4 : (qf == BF16 ? 2 : 1);
  const int tw = (nw / rw) * 64;
  (void)kf;
  // double-buffered tiles, the workgroup's candidate key indices (gather),
  // then one filtering histogram and one flag per wave
  // (16-bit bins for the records of gathered rows)
  return 2 * ((size_t)tw * (D * ke + 16) + (size_t)tw * 8) + ((size_t)gather_cols * 4 + 15) / 16 * 16 +
         (filter ? (size_t)nw * ((filter == 3 ? kFiltBins * 2 : kFiltBins * 4) + 4) : 0);
}

hipError_t launch_score(const ScoreArgs& a, int qf, int kf, int H, int D, int n_col_chunks,
                        hipStream_t st) {
  dim3 grid(a.n_blocks, n_col_chunks);
  if (a.mode == kModeGather && a.kc > kCandLdsMax) return hipErrorInvalidValue;
  const size_t lds = score_lds_bytes(qf, kf, D, a.rw, a.nw, a.filter, a.mode == kModeGather ? a.kc : 0);
  if (lds > kScoreLdsMax) return hipErrorInvalidValue;
  if (qf == F32 && kf == F32) return pick_h<F32, F32>(a, H, D, grid, lds, st);
  if (qf == BF16 && kf == BF16) return pick_h<BF16, BF16>(a, H, D, grid, lds, st);
  if (qf == BF16 && kf == FP8) return pick_h<BF16, FP8>(a, H, D, grid, lds, st);
  if (qf == FP8 && kf == FP8) return pick_h<FP8, FP8>(a, H, D, grid, lds, st);
  return hipErrorInvalidValue;
}

}  // namespace idx
