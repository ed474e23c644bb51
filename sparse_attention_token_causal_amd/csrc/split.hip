// Split-key scan and multi-workgroup select for short row sets on gfx950.
//
// In decode each sequence contributes only the few queries of one
// multi-token-prediction step, but every one of them scans the whole cached
// key history ("ADIndex Restructures Sparse-Attention Indexing with
// Group-Level Distillation", "Why the Indexer Becomes the Bottleneck";
// "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention",
// Abstract: the decode group is the set of queries of one MTP step).  Such a
// scan reads far more key bytes than it has query rows to reuse them on, so
// it is laid out for streaming the keys rather than for tile reuse:
//
//  * a workgroup of 4 waves owns one (sequence, key chunk); the sequence's
//    (query, head) rows - at most 4 queries, 256 rows - are split into
//    64-row waves whose q fragments stay in registers, and the other waves
//    of the workgroup take alternate 32-column steps of the chunk;
//  * the key rows of each 32-column step are copied straight from global
//    memory into an LDS ring of P steps (direct-to-LDS loads, no register
//    staging, several steps in flight); the row-waves of a column group
//    share them, and each lane then reads the half key row of its own MFMA
//    column.  The head dimension is permuted (the same way for q and k,
//    which leaves every dot product unchanged) so that lane half h covers
//    the contiguous half [h*d/2, (h+1)*d/2) of the row;
//  * FP8 keys under bfloat16 q are widened to bfloat16 in registers (exact);
//    FP8 x FP8 runs the f8f6f4 MFMA directly;
//  * the epilogue is the tiled scan's: ReLU, x w (x q scale), head sum in
//    the lane plus one permlane32 swap, key scale, causal mask.
//
// Top-k over rows of 10^5 keys with only a handful of rows needs more than
// one workgroup per row, and no global atomics (same-address atomics from
// many workgroups serialize across the chip's XCDs).  Every eligible score
// also lands in its workgroup's LDS histogram of the top 12 bits of its order
// key, and each workgroup reports a window of that histogram per row; the
// compaction kernel (many workgroups per row) sums the windows, finds the bin
// that holds the row's k-th score and writes every score of its segment in or
// above that bin to the segment's part of the candidate list; the list select
// gathers the segments and ranks the candidates exactly (ties to the lower
// key index).
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace idx {

// gfx9 sched_group_barrier instruction classes
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008;

// Waits until at most n vector-memory operations of this wave are in flight
// (s_waitcnt with the export and LDS counters left at their maxima).
#define IDX_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x70 | 0xF00)

// LDS byte address of a pointer into workgroup memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS copy of BYTES (4 or 16) per lane: lane l's bytes land
// at lds + BYTES * l (lds wave-uniform).  Written as inline assembly so that
// the compiler does not pair every later LDS read with a wait for all
// outstanding copies: the caller waits for them with s_waitcnt itself.  M0
// (which holds the LDS base) is saved and restored; no VGPR is written.
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(const void* src, uint32_t lds) {
  uint32_t saved;
  if constexpr (BYTES == 16)
    __asm__ __volatile__("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                         : "=&s"(saved) : "s"(lds), "v"(src) : "memory");
  else
    __asm__ __volatile__("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
                         : "=&s"(saved) : "s"(lds), "v"(src) : "memory");
}

template <int QF, int KF, int H, int D, int RWN>
__global__ __launch_bounds__(256, 2) void split_scan_kernel(SplitArgs a) {
  constexpr bool F8MMA = (QF == FP8);          // fp8 x fp8 (keys are FP8 too)
  constexpr int KB = (KF == FP8) ? 1 : 2;      // key bytes per element
  constexpr int QB = (QF == FP8) ? 1 : 2;      // q bytes per element
  constexpr int HALF = D / 2;                  // elements per lane half
  constexpr int RB = D * KB;                   // key row bytes
  constexpr int CK = RB / 16;                  // 16-byte chunks per key row
  constexpr int NL = CK / 2;                   // chunks per lane half
  constexpr int SB = split_step_bytes(KB, D);  // bytes per 32-column step
  constexpr int NLD = SB / 1024;               // 1 KiB copies per step
  constexpr int NLDI = split_dma_waves(KB, D, RWN);  // waves issuing them
  constexpr int NLDW = NLD / NLDI;             // copies per issuing wave
  constexpr int P = split_ring_steps(KB, D, RWN);
  constexpr int OPS = split_ops(KB, D, RWN);   // VMEM ops per step, issuing wave
  constexpr int OPS_REST = (KF == FP8) ? 1 : 0;  // ... other waves (scale copy only)
  constexpr int CWN = 4 / RWN;                 // column groups
  constexpr int KSTEP = F8MMA ? 32 : 8;        // elements per lane half per MFMA
  constexpr int NKS = HALF / KSTEP;
  constexpr int QW = 64 / H;                   // queries per wave
  static_assert(P >= 3, "ring depth");
  typedef typename std::conditional<F8MMA, i32x8, bf16x8>::type frag_t;

  // LDS: key ring [CWN][P][SB] | key-scale rings [4 waves][P][64] (FP8) |
  // chunk scores [n_rows][kc] | histograms [n_rows][kSplitBins / 2] (two
  // 16-bit counters per word) | top counted bin [n_rows]
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* ring = smem;
  float* sscale = (float*)(ring + CWN * P * SB);
  float* ssc = sscale + ((KF == FP8) ? 4 * P * 64 : 0);
  uint32_t* shist = (uint32_t*)(ssc + a.n_rows * a.kc);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int l = lane_id(), half = l >> 5, l32 = l & 31;
  const int b = blockIdx.y;
  const int rw = wave % RWN, cw = wave / RWN;

  const int c_begin = (int)blockIdx.x * a.kc;
  int c_end = min(c_begin + a.kc, a.n_k);
  c_end = min(c_end, mode_limit(a.mode, a.q_pos0, a.n_q, a.group, a.block, a.n_rows - 1) + 1);
  if (c_begin >= c_end) {  // the whole workgroup: past every row's prefix
    for (int t = threadIdx.x; t < a.n_rows; t += 256)
      a.wbase[((size_t)b * a.n_rows + t) * a.n_chunks + blockIdx.x] = -1;
    return;
  }
  for (int i = threadIdx.x; i < a.n_rows * (kSplitBins / 2); i += 256) shist[i] = 0u;
  int* s_top = (int*)(shist + a.n_rows * (kSplitBins / 2));  // each row's top counted bin
  if (threadIdx.x < a.n_rows) s_top[threadIdx.x] = -1;

  // ---- resident q fragments and head weights of this wave's 64 rows ----
  // (lane half h holds the elements [h d/2, (h+1) d/2) of each row: the d
  // axis is permuted the same way for the keys)
  const int t_first = rw * QW;
  frag_t afrag[2][NKS];
  float wreg[2][16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int i = 32 * rb + l32;
    const int t = t_first + i / H, h = i % H;
    const bool ok = t < a.n_rows;
    const char* rowp = (const char*)a.q +
                       (((size_t)b * a.n_rows + (ok ? t : 0)) * H + h) * (size_t)D * QB + half * HALF * QB;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      frag_t f = *(const frag_t*)(rowp + ks * KSTEP * QB);
      if (!ok) f = frag_t{};
      afrag[rb][ks] = f;
    }
    // weights of the 16 result rows this lane holds (loads clamped to valid
    // rows, all in flight together; rows past the set weigh 0)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ri = 32 * rb + 8 * (v / 4) + 4 * half + (v % 4);
      const int tt = t_first + ri / H, hh = ri % H;
      const size_t fr = (size_t)b * a.n_rows + min(tt, a.n_rows - 1);
      wreg[rb][v] = a.w[fr * H + hh] * (QF == FP8 ? a.q_scale[fr] : 1.f);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ri = 32 * rb + 8 * (v / 4) + 4 * half + (v % 4);
      if (t_first + ri / H >= a.n_rows) wreg[rb][v] = 0.f;
    }
  }
  // (the histograms' zeroing and the q loads are complete at the barrier
  // after the ring's first copies, so both latencies overlap)

  // ---- steps: group cw takes steps c_begin + 32 * (cw + CWN * i) ----
  const int n_steps = (c_end - c_begin + 31) / 32;
  const int n_iter = (n_steps + CWN - 1) / CWN;  // the same for every wave (barriers)
  const int n_my = cw < n_steps ? (n_steps - cw + CWN - 1) / CWN : 0;
  const bool has_rows = t_first < a.n_rows;
  const char* kseq = (const char*)a.k + (size_t)b * a.n_k * RB;
  const float* kscl = (KF == FP8) ? a.k_scale + (size_t)b * a.n_k : nullptr;
  char* gring = ring + cw * P * SB;
  float* wscale = sscale + wave * P * 64;

  // Direct-to-LDS copies of step i into ring slot i % P.  Copy dd of a step
  // fills bytes [1024 dd, 1024 dd + 1024) of the slot, lane l the 16 bytes at
  // 16 l: key r = p / CK, chunk position cp = p % CK (p = 64 dd + l), which
  // holds the key's chunk cp ^ (r % CK) (an XOR swizzle: the 16-byte reads of
  // 8 consecutive keys hit distinct bank groups).  Columns past the chunk
  // copy its last key (in bounds; masked later).  Every wave also copies the
  // 32 key scales of its own steps into its scale ring (FP8 keys).
  auto issue = [&](int i) {
    const int slot = i % P;
    const int col0 = c_begin + 32 * (cw + CWN * i);
    if (rw < NLDI) {
#pragma unroll
      for (int d = 0; d < NLDW; ++d) {
        const int dd = rw * NLDW + d;
        const int p = dd * 64 + l;
        const int r = p / CK, cp = p % CK;
        const int key = min(col0 + r, c_end - 1);
        copy_to_lds<16>(kseq + (size_t)key * RB + 16 * (cp ^ (r % CK)),
                        __builtin_amdgcn_readfirstlane(lds_addr(gring + slot * SB + dd * 1024)));
      }
    }
    if constexpr (KF == FP8) {
      const int key = min(col0 + l32, c_end - 1);
      copy_to_lds<4>(kscl + key, __builtin_amdgcn_readfirstlane(lds_addr(wscale + slot * 64)));
    }
  };
  // this lane's half key row of step i: NL 16-byte chunks
  auto read_keys = [&](int i, i32x4* raw) {
    const char* row = gring + (i % P) * SB + l32 * RB;
#pragma unroll
    for (int u = 0; u < NL; ++u) raw[u] = *(const i32x4*)(row + 16 * ((half * NL + u) ^ (l32 % CK)));
  };
  auto bfrag = [&](const i32x4* r, int ks) -> frag_t {
    if constexpr (F8MMA) {
      const i32x4 x = r[2 * ks], y = r[2 * ks + 1];
      return frag_t{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    } else if constexpr (KF == FP8) {
      const i32x4 x = r[ks / 2];
      uint32_t o0, o1, o2, o3;
      fp8x4_to_bf16x4((uint32_t)x[(ks % 2) * 2], o0, o1);
      fp8x4_to_bf16x4((uint32_t)x[(ks % 2) * 2 + 1], o2, o3);
      return __builtin_bit_cast(frag_t, (i32x4{(int)o0, (int)o1, (int)o2, (int)o3}));
    } else {
      return __builtin_bit_cast(frag_t, r[ks]);
    }
  };
  auto mma = [&](frag_t x, frag_t y, f32x16 c) -> f32x16 {
    if constexpr (F8MMA)
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
  };

  // last visible key of each of this wave's queries (-1 past the row set)
  int qlim[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi)
    qlim[qi] = t_first + qi < a.n_rows ? mode_limit(a.mode, a.q_pos0, a.n_q, a.group, a.block, t_first + qi) : -1;

  // each lane's highest counted bin per row (the row's histogram window ends
  // at the maximum over the workgroup: no scan of the histogram at the end)
  int topb[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) topb[qi] = -1;
  // ---- epilogue of step i: ReLU, x w, head sum, key scale, mask -> LDS scores + histogram ----
  auto epilogue = [&](const f32x16* acc, int i, float ksc) {
    const int col_raw = c_begin + 32 * (cw + CWN * i) + l32;
    const int col = min(col_raw, c_end - 1);  // the column whose key this lane used
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if ((32 * rb + 8 * (v / 4)) / H == qi) {
            // ReLU as an integer max of the bits: negative floats (and -0)
            // are negative integers, so they become +0 (one VALU op, no
            // NaN canonicalisation; the MFMA results are finite)
            const float r = __int_as_float(max(__float_as_int(acc[rb][v]), 0));
            if (v & 1)
              p1 = __builtin_fmaf(wreg[rb][v], r, p1);
            else
              p0 = __builtin_fmaf(wreg[rb][v], r, p0);
          }
      const float p = p0 + p1;
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
      const float tot = p + __uint_as_float(half ? sw[0] : sw[1]);
      const int t = t_first + qi;
      // Both halves hold the total; a lane past the chunk computed the score
      // of the chunk's last column and stores it there again (same value).
      // Only half (qi % 2)'s lanes inside the chunk count.
      if (QW == 1 || t < a.n_rows) {
        const bool ok = col <= qlim[qi];
        const float val = ok ? (KF == FP8 ? tot * ksc : tot) : neg_inf();
        ssc[t * a.kc + (col - c_begin)] = val;
        const uint32_t bin = order_key(val) >> kSplitShift;
        const bool count = ok && half == (qi & 1) && col_raw < c_end;
        atomicAdd(&shist[t * (kSplitBins / 2) + (bin >> 1)], count ? (1u << (16 * (bin & 1))) : 0u);
        topb[qi] = count ? max(topb[qi], (int)bin) : topb[qi];
      }
    }
  };

  // ---- pipelined scan ----
  // Iteration i: wait for this wave's copies of step i + 1, barrier (every
  // copy of step i + 1 has landed, every read of the slot refilled next is
  // done), copy step i + P - 1 into the slot step i - 1 used, read step
  // i + 1's keys from LDS into registers, then the MFMAs of step i
  // (accumulator set i % 2) interleaved with the epilogue of step i - 1.
  // The body is one basic block: a step past this group's end computes on
  // its clamped keys (the chunk's last column, stored again with the same
  // value and not counted), and a wave without rows computes nothing.  No
  // global store is issued inside the loop, so the vector-memory counter
  // only counts these copies (and they complete in order).
  constexpr int NM = 2 * NKS;                 // MFMAs per step
  constexpr int VPM = NM >= 16 ? 6 : 96 / NM;  // VALU ops placed after each
  f32x16 acc[2][2];
  i32x4 raw[2][NL];
  float ksc[2] = {1.f, 1.f};
  auto wait_step = [&](auto after_c) {  // at most `after` steps of copies still in flight
    constexpr int AFTER = decltype(after_c)::value;
    if (rw < NLDI)
      IDX_WAIT_VM(AFTER * OPS);
    else
      IDX_WAIT_VM(AFTER * OPS_REST);
  };
  auto iteration = [&](auto par_c, auto first_c, int i) {
    constexpr int PAR = decltype(par_c)::value;  // i % 2
    constexpr bool FIRST = decltype(first_c)::value;
    wait_step(std::integral_constant<int, P - 3>{});
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");  // no LDS access moves above the barrier
    issue(i + P - 1);
    if (has_rows) {
      const float kprev = ksc[1 - PAR];  // step i - 1's scale; the slot takes step i + 1's
      read_keys(i + 1, raw[1 - PAR]);
      if constexpr (KF == FP8) ksc[1 - PAR] = wscale[((i + 1) % P) * 64 + l32];
      f32x16* c = acc[PAR];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const frag_t bf = bfrag(raw[PAR], ks);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) c[rb] = mma(afrag[rb][ks], bf, ks == 0 ? f32x16{} : c[rb]);
      }
      if constexpr (!FIRST) epilogue(acc[1 - PAR], i - 1, kprev);
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, VPM, 0);
      }
    }
  };
  for (int i = 0; i < P - 1; ++i) issue(i);
  wait_step(std::integral_constant<int, P - 2>{});  // step 0 landed
  __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): histograms zeroed
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
  if (has_rows) {
    read_keys(0, raw[0]);
    if constexpr (KF == FP8) ksc[0] = wscale[l32];
  }
  iteration(std::integral_constant<int, 0>{}, std::true_type{}, 0);
  int i = 1;
  for (; i + 1 < n_iter; i += 2) {
    iteration(std::integral_constant<int, 1>{}, std::false_type{}, i);
    iteration(std::integral_constant<int, 0>{}, std::false_type{}, i + 1);
  }
  if (i < n_iter) iteration(std::integral_constant<int, 1>{}, std::false_type{}, i);
  if (has_rows) {  // the last step's epilogue
    if ((n_iter - 1) & 1)
      epilogue(acc[1], n_iter - 1, ksc[1]);
    else
      epilogue(acc[0], n_iter - 1, ksc[0]);
  }
  if (has_rows) {
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      int m = topb[qi];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, kWave));
      if (l == 0 && t_first + qi < a.n_rows) atomicMax(&s_top[t_first + qi], m);
    }
  }
  IDX_WAIT_VM(0);   // the copies issued past the last step have landed too
  __syncthreads();  // every score and count in LDS

  // ---- chunk scores to global memory (coalesced) ----
  const int width = c_end - c_begin;
  for (int t = 0; t < a.n_rows; ++t) {
    float* dst = a.out + ((size_t)b * a.n_rows + t) * a.n_k + c_begin;
    for (int j = threadIdx.x; j < width; j += 256) dst[j] = ssc[t * a.kc + j];
  }

  // ---- report each row's histogram window: the kSplitWin bins up to its top non-empty one ----
  for (int t = wave; t < a.n_rows; t += 4) {
    const uint32_t* hr = shist + t * (kSplitBins / 2);
    const int m = s_top[t];
    const int wb = m < 0 ? -1 : max(m - kSplitWin + 1, 0);
    const size_t slot = ((size_t)b * a.n_rows + t) * a.n_chunks + blockIdx.x;
    if (l == 0) a.wbase[slot] = wb;
    for (int j = l; j < kSplitWin; j += kWave) {
      const int bin = wb + j;
      a.win[slot * kSplitWin + j] = wb < 0 ? 0u : (hr[bin >> 1] >> (16 * (bin & 1))) & 0xFFFFu;
    }
  }
}
#undef IDX_WAIT_VM

// ---- compaction: threshold bin from the chunks' histogram windows, then
// every score of this segment in or above it, in column order, into the
// segment's slots of the candidate list ----
//
// A window covers the bins of its chunk from kSplitWin below the chunk's top
// non-empty bin; counts below a window are dropped, so the summed histogram
// can only undercount, the threshold bin only comes out lower, and the list
// can only grow: it always holds the row's top-k.  The segment's first batch
// of scores is loaded together with the windows (it does not depend on the
// threshold); the first segment's workgroup records the row's threshold bin
// for the select.
__global__ __launch_bounds__(256) void split_compact_kernel(CompactArgs a) {
  __shared__ uint32_t hist[kSplitBins];
  __shared__ int wtot[4];
  __shared__ int s_thr;
  const int row = blockIdx.y;
  const int t = row % a.n_rows;
  const int len = min(mode_limit(a.mode, a.q_pos0, a.n_q, a.group, a.block, t) + 1, a.n_k);
  const int s0 = (int)blockIdx.x * a.seg, s1 = min(s0 + a.seg, len);
  const int tid = threadIdx.x, wave = tid / kWave, l = lane_id();
  int* segcnt = a.segcnt + (size_t)row * a.n_segs + blockIdx.x;
  if (s0 >= s1) {
    if (tid == 0) *segcnt = 0;
    return;
  }
  const int need = min(a.topk, len);

  // the first batch of the segment's scores, in flight with the window loads
  constexpr int kBatch = 16 * 256;
  const float* srow = a.scores + (size_t)row * a.n_k;
  float v[16];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = srow[min(c0 + u * 256 + tid, s1 - 1)];
  };
  load_batch(s0);

  for (int i = tid; i < kSplitBins; i += 256) hist[i] = 0u;
  if (tid == 0) s_thr = 0;
  __syncthreads();
  const int* wb = a.wbase + (size_t)row * a.n_chunks;
  const uint32_t* wn = a.win + (size_t)row * a.n_chunks * kSplitWin;
  // runs of four window entries per thread (16-byte loads; a run never
  // crosses a window), eight runs per thread per batch: all loads in flight
  // together (one batch for up to 64 chunks)
  const int n_e = a.n_chunks * kSplitWin;
  static_assert(kSplitWin % 4 == 0, "runs of four entries");
  for (int e0 = 0; e0 < n_e; e0 += 8 * 4 * 256) {
    uint4 cv[8];
    int bv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = min(e0 + 4 * (u * 256 + tid), n_e - 4);
      bv[u] = wb[e / kSplitWin];
      cv[u] = *(const uint4*)(wn + e);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + 4 * (u * 256 + tid);
      if (e < n_e && bv[u] >= 0) {
        const uint32_t c4[4] = {cv[u].x, cv[u].y, cv[u].z, cv[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c4[q]) atomicAdd(&hist[bv[u] + e % kSplitWin + q], c4[q]);
      }
    }
  }
  __syncthreads();

  // Block-wide exclusive prefix sum of one int per thread (+ the total).
  auto block_scan = [&](int x, int* total) {
    const int incl = wave_incl_scan(x);
    if (l == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += w < wave ? wtot[w] : 0;
      tot += wtot[w];
    }
    __syncthreads();
    *total = tot;
    return before + incl - x;
  };

  // thread i owns bins [16 i, 16 i + 16): the threshold is the highest bin
  // with at least `need` counts at or above it (0 when the sum falls short)
  static_assert(kSplitBins == 16 * 256, "16 bins per thread of the 256");
  uint32_t c[16];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    c[j] = hist[16 * tid + j];
    mine += (int)c[j];
  }
  int total;
  const int before = block_scan(mine, &total);
  int above = total - before - mine;  // counts in the bins of higher threads
  if (above < need && above + mine >= need) {
    for (int j = 15; j >= 0; --j) {
      if (above + (int)c[j] >= need) {
        s_thr = 16 * tid + j;
        break;
      }
      above += (int)c[j];
    }
  }
  __syncthreads();
  const uint32_t thr = (uint32_t)s_thr;

  if (blockIdx.x == 0 && tid == 0) a.thr[row] = (int)thr;

  float* cv = a.cval + (size_t)row * a.n_k + s0;
  int* ci = a.cidx + (size_t)row * a.n_k + s0;
  int filled = 0;
  for (int c0 = s0; c0 < s1; c0 += kBatch) {
    if (c0 != s0) load_batch(c0);
    uint32_t pm = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int col = c0 + u * 256 + tid;
      pm |= (uint32_t)(col < s1 && (order_key(v[u]) >> kSplitShift) >= thr) << u;
    }
    int tot;
    int o = filled + block_scan(__builtin_popcount(pm), &tot);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if ((pm >> u) & 1u) {
        cv[o] = v[u];
        ci[o] = c0 + u * 256 + tid;
        ++o;
      }
    }
    filled += tot;
  }
  if (tid == 0) *segcnt = filled;
}

template <int QF, int KF, int H, int D, int RWN>
static hipError_t launch_split_t(const SplitArgs& a, int B, int chunks, hipStream_t st) {
  static bool attr_set = false;  // once per instantiation: allow more than 64 KiB of LDS
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)split_scan_kernel<QF, KF, H, D, RWN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSplitLdsMax);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t lds = split_lds_bytes(KF == FP8 ? 1 : 2, D, RWN, a.n_rows, a.kc);
  if (lds > kSplitLdsMax || a.kc % (32 * (4 / RWN)) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((split_scan_kernel<QF, KF, H, D, RWN>), dim3(chunks, B), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int QF, int KF, int H, int D>
static hipError_t split_pick_rwn(const SplitArgs& a, int B, int chunks, hipStream_t st) {
  if (a.rwn == 1) return launch_split_t<QF, KF, H, D, 1>(a, B, chunks, st);
  if constexpr (H >= 32) {
    if (a.rwn == 2) return launch_split_t<QF, KF, H, D, 2>(a, B, chunks, st);
  }
  if constexpr (H == 64) {
    if (a.rwn == 4) return launch_split_t<QF, KF, H, D, 4>(a, B, chunks, st);
  }
  return hipErrorInvalidValue;
}

template <int QF, int KF, int H>
static hipError_t split_pick_d(const SplitArgs& a, int D, int B, int chunks, hipStream_t st) {
  if (D == 64) return split_pick_rwn<QF, KF, H, 64>(a, B, chunks, st);
  if (D == 128) return split_pick_rwn<QF, KF, H, 128>(a, B, chunks, st);
  return hipErrorInvalidValue;
}

template <int QF, int KF>
static hipError_t split_pick_h(const SplitArgs& a, int H, int D, int B, int chunks, hipStream_t st) {
  if (H == 16) return split_pick_d<QF, KF, 16>(a, D, B, chunks, st);
  if (H == 32) return split_pick_d<QF, KF, 32>(a, D, B, chunks, st);
  if (H == 64) return split_pick_d<QF, KF, 64>(a, D, B, chunks, st);
  return hipErrorInvalidValue;
}

hipError_t launch_split_scan(const SplitArgs& a, int qf, int kf, int H, int D, int B, int chunks,
                             hipStream_t st) {
  if (qf == BF16 && kf == BF16) return split_pick_h<BF16, BF16>(a, H, D, B, chunks, st);
  if (qf == BF16 && kf == FP8) return split_pick_h<BF16, FP8>(a, H, D, B, chunks, st);
  if (qf == FP8 && kf == FP8) return split_pick_h<FP8, FP8>(a, H, D, B, chunks, st);
  return hipErrorInvalidValue;
}

hipError_t launch_split_compact(const CompactArgs& a, int rows, hipStream_t st) {
  hipLaunchKernelGGL(split_compact_kernel, dim3(a.n_segs, rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace idx
