// Per-row exact top-k select for gfx950.
//
// One workgroup per row of scores.  The order is (score descending, key
// index ascending) with exact equality as a tie and -0 == +0 ("PIVOT:
// Efficient Query-Group Indexing for Token-Level Sparse Attention",
// Abstract: each query keeps its own top-k of the scanned or re-scored
// keys; the tie rule is the reading given in the library header).
//
// Method: scores are mapped to order-preserving 32-bit keys; a most-
// significant-digit-first radix select (four 8-bit digits) finds the key tau
// of the k-th entry and how many entries equal to tau still belong to the
// top-k.  If only part of the tie class is taken, a second radix select
// (ascending, over the key indices of the tied entries) finds the largest
// admitted index.  A final ordered compaction (wave ballot + popcount prefix
// counts) writes the winners in column order and pads the row with -1.
// Histograms live in LDS in eight copies (lane & 7) to spread same-bin
// atomics; rows of up to 32768 keys are cached in LDS, longer rows are
// re-read from global memory on each pass.
#include "common.hpp"
#include "kernels.hpp"

namespace idx {

constexpr int kCopies = 8;
constexpr int kCopyStride = 257;

struct SelectShared {
  uint32_t hist[kCopies * kCopyStride];
  uint32_t bins[256];
  int wsum[kSelectThreads / kWave];
  int scan[4];
  uint32_t sel_digit;
  int sel_before;
  int total;
};

// Inclusive prefix over threads 0..255 of v (other threads get 0).  All
// threads of the block must call it.
__device__ __forceinline__ int scan256(int v, SelectShared& sh) {
  const int w = threadIdx.x / kWave;
  int x = 0;
  if (threadIdx.x < 256) {
    x = wave_incl_scan(v);
    if (lane_id() == kWave - 1) sh.scan[w] = x;
  }
  __syncthreads();
  if (threadIdx.x < 256)
    for (int i = 0; i < w; ++i) x += sh.scan[i];
  __syncthreads();
  return x;
}

__device__ __forceinline__ void clear_hist(SelectShared& sh) {
  for (int i = threadIdx.x; i < kCopies * kCopyStride; i += kSelectThreads) sh.hist[i] = 0;
}

// Sum the histogram copies into bins[]; then pick the digit that holds rank
// `rank` (1-based), counting from the largest digit when `descending`, from
// the smallest otherwise.  Returns the digit; *before = entries ranked
// ahead of that digit.
__device__ uint32_t pick_digit(SelectShared& sh, int rank, bool descending, int* before) {
  __syncthreads();
  if (threadIdx.x < 256) {
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < kCopies; ++c) s += sh.hist[c * kCopyStride + threadIdx.x];
    sh.bins[threadIdx.x] = s;
  }
  __syncthreads();
  const int d = descending ? 255 - (int)threadIdx.x : (int)threadIdx.x;
  const int cnt = (threadIdx.x < 256) ? (int)sh.bins[d] : 0;
  const int incl = scan256(cnt, sh);
  if (threadIdx.x < 256) {
    const int excl = incl - cnt;
    if (excl < rank && rank <= incl) {
      sh.sel_digit = (uint32_t)d;
      sh.sel_before = excl;
    }
  }
  __syncthreads();
  *before = sh.sel_before;
  return sh.sel_digit;
}

__device__ __forceinline__ int row_length(const SelectArgs& a, int r) {
  if (a.mode == kModeGather) return a.n_cols;
  const int lim = (a.mode == kModeProxy) ? a.q_pos0 + min((r + 1) * a.group, a.n_q) - 1
                                         : a.q_pos0 + r;
  return min(lim + 1, a.n_cols);
}

__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a, int cache_cap) {
  __shared__ SelectShared sh;
  extern __shared__ uint32_t skeys[];

  const long long frow = a.row0 + blockIdx.x;
  const int b = (int)(frow / a.n_rows), r = (int)(frow % a.n_rows);
  const float* row = a.scores + (long long)blockIdx.x * a.ld;
  int* out = a.out + frow * (long long)a.topk;
  const int* crow = nullptr;
  if (a.mode == kModeGather) {
    const int n_g = (a.n_q + a.group - 1) / a.group;
    crow = a.cand + ((long long)b * n_g + r / a.group) * a.n_cols;
  }
  const int len = row_length(a, r);
  const bool cached = len <= cache_cap;
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int copy = lane & (kCopies - 1);

  auto key_at = [&](int c) -> uint32_t {
    if (cached) return skeys[c];
    const float v = row[c];
    return v == neg_inf() ? kKeyExcluded : order_key(v);
  };
  auto index_at = [&](int c) -> int { return crow ? crow[c] : c; };

  // ---- load (and cache) the keys, count the eligible ones ----
  int nv = 0;
  for (int c = tid; c < len; c += kSelectThreads) {
    const float v = row[c];
    const uint32_t k = v == neg_inf() ? kKeyExcluded : order_key(v);
    if (cached) skeys[c] = k;
    nv += (k != kKeyExcluded);
  }
  nv = wave_sum(nv);
  if (lane == 0) sh.wsum[wave] = nv;
  __syncthreads();
  int n_valid = 0;
  for (int i = 0; i < kSelectThreads / kWave; ++i) n_valid += sh.wsum[i];
  __syncthreads();

  // ---- threshold: winners are key > tau, or key == tau with index <= idx_thr ----
  uint32_t tau = kKeyExcluded;
  int idx_thr = -1;
  if (n_valid > a.topk) {
    uint32_t prefix = 0, pmask = 0;
    int rank = a.topk, before = 0, eq_count = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      clear_hist(sh);
      __syncthreads();
      for (int c = tid; c < len; c += kSelectThreads) {
        const uint32_t k = key_at(c);
        if (k != kKeyExcluded && (k & pmask) == prefix)
          atomicAdd(&sh.hist[copy * kCopyStride + ((k >> shift) & 255u)], 1u);
      }
      const uint32_t d = pick_digit(sh, rank, true, &before);
      eq_count = (int)sh.bins[d];
      rank -= before;
      prefix |= d << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    tau = prefix;
    if (rank == eq_count) {
      idx_thr = 0x7FFFFFFF;
    } else {
      // the rank-th smallest key index among the entries equal to tau
      uint32_t ip = 0, im = 0;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        clear_hist(sh);
        __syncthreads();
        for (int c = tid; c < len; c += kSelectThreads) {
          if (key_at(c) == tau) {
            const uint32_t ix = (uint32_t)index_at(c);
            if ((ix & im) == ip) atomicAdd(&sh.hist[copy * kCopyStride + ((ix >> shift) & 255u)], 1u);
          }
        }
        const uint32_t d = pick_digit(sh, rank, false, &before);
        rank -= before;
        ip |= d << shift;
        im |= 255u << shift;
        __syncthreads();
      }
      idx_thr = (int)ip;
    }
  }

  // ---- ordered compaction of the winners ----
  int base = 0;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int c0 = 0; c0 < len; c0 += kSelectThreads) {
    const int c = c0 + tid;
    bool win = false;
    int ix = 0;
    if (c < len) {
      const uint32_t k = key_at(c);
      if (k != kKeyExcluded && k > tau) {
        win = true;
        ix = index_at(c);
      } else if (k != kKeyExcluded && k == tau) {
        ix = index_at(c);
        win = ix <= idx_thr;
      }
    }
    const unsigned long long m = __ballot(win);
    if (lane == 0) sh.wsum[wave] = __popcll(m);
    __syncthreads();
    int off = base, total = 0;
    for (int i = 0; i < kSelectThreads / kWave; ++i) {
      if (i < wave) off += sh.wsum[i];
      total += sh.wsum[i];
    }
    if (win) out[off + __popcll(m & lt)] = ix;
    base += total;
    __syncthreads();
  }
  for (int i = base + tid; i < a.topk; i += kSelectThreads) out[i] = -1;
}

hipError_t launch_select(const SelectArgs& a, int n_launch_rows, hipStream_t st) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 16 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int cap = a.n_cols < kSelectCache ? a.n_cols : kSelectCache;
  hipLaunchKernelGGL(select_kernel, dim3(n_launch_rows), dim3(kSelectThreads),
                     (size_t)cap * sizeof(uint32_t), st, a, cap);
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
