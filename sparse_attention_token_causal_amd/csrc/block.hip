// Block-mean candidate routing for gfx950: block representatives and the
// expansion of the routed blocks into a Refine candidate list.
//
// "AttentionIndex Architecture ...", "Why Positional Blocks Lose Recall":
// two-stage selection routes each query to contiguous blocks of keys ranked
// by a mean-pooled representative, then runs the native indexer only on the
// keys of the kept blocks ("Worked Example: Blocks Lose, Clusters Win" keeps
// the best two blocks).  Here the router is the group's PIVOT proxy, the
// block score is the indexer form applied to the block mean (the scan itself
// is the proxy scan with block-mean "keys"), a block is routable for a group
// only when it lies wholly inside the prefix of the group's last member, and
// the keys of the trailing partial block are always candidates.
#include "common.hpp"
#include "kernels.hpp"

namespace idx {

// One workgroup per (block, sequence); thread e < D sums element e of the
// block's real keys in token order (float32), divides by the key count and
// stores bfloat16 (nearest, ties to even) for BF16/FP8 keys, float32 for F32
// keys.  HBM-bound: every key element is read once, coalesced along d.
template <int KF>
__global__ __launch_bounds__(128) void block_mean_kernel(const void* k, const float* k_scale, int n_k,
                                                         int D, int block, void* kbar) {
  const int j = blockIdx.x, b = blockIdx.y;
  const int n_b = (n_k + block - 1) / block;
  const int s0 = j * block, s1 = min(s0 + block, n_k);
  const float n = (float)(s1 - s0);
  const size_t orow = (size_t)b * n_b + j;
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float acc = 0.f;
    for (int s = s0; s < s1; ++s) {
      const size_t off = ((size_t)b * n_k + s) * D + e;
      float v;
      if (KF == F32) {
        v = ((const float*)k)[off];
      } else if (KF == BF16) {
        v = __uint_as_float((uint32_t)((const uint16_t*)k)[off] << 16);
      } else {
        v = fp8_to_f32(((const uint8_t*)k)[off]) * k_scale[(size_t)b * n_k + s];
      }
      acc += v;
    }
    const float m = acc / n;
    if (KF == F32)
      ((float*)kbar)[orow * D + e] = m;
    else
      ((uint16_t*)kbar)[orow * D + e] = f32_to_bf16_rne(m);
  }
}

hipError_t launch_block_means(const void* k, const float* k_scale, int B, int n_k, int D, int kf,
                              int block, void* kbar, hipStream_t st) {
  dim3 grid((n_k + block - 1) / block, B);
  if (kf == F32)
    hipLaunchKernelGGL(block_mean_kernel<F32>, grid, dim3(128), 0, st, k, k_scale, n_k, D, block, kbar);
  else if (kf == BF16)
    hipLaunchKernelGGL(block_mean_kernel<BF16>, grid, dim3(128), 0, st, k, k_scale, n_k, D, block, kbar);
  else
    hipLaunchKernelGGL(block_mean_kernel<FP8>, grid, dim3(128), 0, st, k, k_scale, n_k, D, block, kbar);
  return hipGetLastError();
}

// One workgroup per (group, sequence).  Slot i of the candidate row (width
// (n_sel + 1) * block): the u-th key of the (i / block)-th routed block while
// routed blocks last, then the keys of the trailing partial block of the
// group's prefix, then -1.  The routed blocks come first in `sel` (the select
// pads its rows at the end), so their number is the count of valid entries.
// Each thread issues the loads of eight slots before storing them.
constexpr int kExpandBatch = 8;

__global__ __launch_bounds__(256) void block_expand_kernel(const int* sel, int n_q, int q_pos0, int group,
                                                           int block, int n_sel, int* cand) {
  __shared__ int s_cnt[4];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n_g = (n_q + group - 1) / group;
  const int* srow = sel + ((size_t)b * n_g + g) * n_sel;
  int cnt = 0;
  for (int i = tid; i < n_sel; i += 256) cnt += srow[i] >= 0 ? 1 : 0;
  cnt = wave_sum(cnt);
  if (lane_id() == 0) s_cnt[tid / kWave] = cnt;
  __syncthreads();
  const int n_routed = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
  const int last = mode_limit(kModeProxy, q_pos0, n_q, group, block, g);  // pos(t_last)
  const int n_full = (last + 1) / block;
  const int tail = last + 1 - n_full * block;
  const int width = (n_sel + 1) * block;
  int* crow = cand + ((size_t)b * n_g + g) * width;
  for (int i0 = 0; i0 < width; i0 += kExpandBatch * 256) {
    int key[kExpandBatch];
#pragma unroll
    for (int j = 0; j < kExpandBatch; ++j) {
      const int i = i0 + j * 256 + tid;
      const int blk = i / block, u = i % block;
      key[j] = -1;
      if (i < width) {
        if (blk < n_routed)
          key[j] = srow[blk] * block + u;
        else if (i - n_routed * block < tail)
          key[j] = n_full * block + (i - n_routed * block);
      }
    }
#pragma unroll
    for (int j = 0; j < kExpandBatch; ++j) {
      const int i = i0 + j * 256 + tid;
      if (i < width) crow[i] = key[j];
    }
  }
}

hipError_t launch_block_expand(const int* sel, int B, int n_q, int q_pos0, int group, int block,
                               int n_sel, int* cand, hipStream_t st) {
  dim3 grid((n_q + group - 1) / group, B);
  hipLaunchKernelGGL(block_expand_kernel, grid, dim3(256), 0, st, sel, n_q, q_pos0, group, block, n_sel, cand);
  return hipGetLastError();
}

}  // namespace idx
