// PIVOT proxy construction and Reuse broadcast for gfx950.
//
// "PIVOT: Efficient Query-Group Indexing for Token-Level Sparse Attention",
// Abstract: a group of nearby queries is aggregated into a single proxy
// query (read here as the mean of the members' real q and of their head
// weights w); PIVOT-Reuse shares the proxy's top-k with every member.  A
// member keeps only the shared entries inside its own causal prefix and the
// freed slots are not refilled.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace idx {

// One workgroup per (group, sequence, part of the (head, dim) row): the row
// is split over gridDim.z workgroups when there are too few groups to fill
// the chip (decode: one group per sequence).  Sums run over the members in
// token order in float32, then divide by the member count; the proxy q is
// stored as bfloat16 (nearest, ties to even) for BF16/FP8 inputs and as
// float32 for F32 inputs, the proxy w as float32.  HBM-bound: every q
// element is read once; each thread owns 16-byte chunks of the row
// (coalesced across the workgroup) and loads four members at a time (a
// group of fewer members issues all its loads at once).
template <int QF>
__global__ __launch_bounds__(256) void proxy_build_kernel(const void* q, const float* q_scale,
                                                          const float* w, int n_q, int H, int D,
                                                          int group, void* pq, float* pw) {
  constexpr int EB = QF == F32 ? 4 : (QF == BF16 ? 2 : 1);  // bytes per q element
  constexpr int VEC = 16 / EB;                              // elements per 16-byte chunk
  const int g = blockIdx.x, b = blockIdx.y;
  const int n_g = (n_q + group - 1) / group;
  const int t0 = g * group, t1 = min(t0 + group, n_q);
  const float n = (float)(t1 - t0);
  const size_t HD = (size_t)H * D;
  const size_t prow = (size_t)b * n_g + g;
  const char* qb = (const char*)q + (size_t)b * n_q * HD * EB;
  auto decode = [&](const i32x4& raw, int t, float* v) {
    if constexpr (QF == F32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __int_as_float(raw[i]);
    } else if constexpr (QF == BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float((uint32_t)raw[i] << 16);
        v[2 * i + 1] = __uint_as_float((uint32_t)raw[i] & 0xFFFF0000u);
      }
    } else {
      const float sc = q_scale[(size_t)b * n_q + t];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = fp8_to_f32(((uint32_t)raw[i / 4] >> (8 * (i % 4))) & 0xFFu) * sc;
    }
  };
  for (size_t ch = (size_t)blockIdx.z * blockDim.x + threadIdx.x; ch * VEC < HD;
       ch += (size_t)gridDim.z * blockDim.x) {
    float s[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) s[i] = 0.f;
    for (int t = t0; t < t1; t += 4) {
      // four members' loads in flight (past the group's end: its last member
      // again, not added)
      i32x4 raw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        raw[u] = *(const i32x4*)(qb + ((size_t)min(t + u, t1 - 1) * HD + ch * VEC) * EB);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (t + u < t1) {
          float v[VEC];
          decode(raw[u], t + u, v);
#pragma unroll
          for (int i = 0; i < VEC; ++i) s[i] += v[i];
        }
      }
    }
    const size_t o = prow * HD + ch * VEC;
    if constexpr (QF == F32) {
      *(float4*)((float*)pq + o) = make_float4(s[0] / n, s[1] / n, s[2] / n, s[3] / n);
    } else {
      uint32_t packed[VEC / 2];
#pragma unroll
      for (int i = 0; i < VEC / 2; ++i)
        packed[i] = (uint32_t)f32_to_bf16_rne(s[2 * i] / n) | ((uint32_t)f32_to_bf16_rne(s[2 * i + 1] / n) << 16);
#pragma unroll
      for (int i = 0; i < VEC / 8; ++i)
        *(i32x4*)((uint16_t*)pq + o + 8 * i) =
            i32x4{(int)packed[4 * i], (int)packed[4 * i + 1], (int)packed[4 * i + 2], (int)packed[4 * i + 3]};
    }
  }
  for (int h = threadIdx.x; h < (blockIdx.z == 0 ? H : 0); h += blockDim.x) {
    float s = 0.f;  // member order, eight loads in flight
    int t = t0;
    for (; t + 8 <= t1; t += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = w[((size_t)b * n_q + t + u) * H + h];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += x[u];
    }
    for (; t < t1; ++t) s += w[((size_t)b * n_q + t) * H + h];
    pw[prow * H + h] = s / n;
  }
}

hipError_t launch_proxy_build(const void* q, const float* q_scale, const float* w, int B, int n_q,
                              int H, int D, int qf, int group, void* pq, float* pw,
                              hipStream_t st) {
  const int n_g = (n_q + group - 1) / group;
  // parts of the (head, dim) row: about 256 workgroups in all, each thread at
  // least one 16-byte chunk
  const long long chunks = (long long)H * D * (qf == F32 ? 4 : (qf == BF16 ? 2 : 1)) / 16;
  long long parts = std::max(1LL, 256LL / ((long long)n_g * B));
  parts = std::min(parts, std::max(1LL, chunks / 256));
  dim3 grid(n_g, B, (unsigned)parts);
  if (qf == F32)
    hipLaunchKernelGGL(proxy_build_kernel<F32>, grid, dim3(256), 0, st, q, q_scale, w, n_q, H, D, group, pq, pw);
  else if (qf == BF16)
    hipLaunchKernelGGL(proxy_build_kernel<BF16>, grid, dim3(256), 0, st, q, q_scale, w, n_q, H, D, group, pq, pw);
  else
    hipLaunchKernelGGL(proxy_build_kernel<FP8>, grid, dim3(256), 0, st, q, q_scale, w, n_q, H, D, group, pq, pw);
  return hipGetLastError();
}

// One wave per query: filter the group's shared list to the query's causal
// prefix and compact it in order (ballot + popcount prefix), then pad.
// HBM-write-bound: every member writes a full row of topk indices.  The list
// is read in tiles of kReuseChunks x 64 entries whose loads are all issued
// before the first ballot, so a row costs about one load latency per tile
// rather than one per 64 entries (the lists are shared by the group's
// members and come from the L2).
constexpr int kReuseChunks = 16;

__global__ __launch_bounds__(256) void reuse_kernel(const int* ptop, int n_q, int q_pos0, int group,
                                                    int topk, int* out) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int t = blockIdx.x * (256 / kWave) + wave, b = blockIdx.y;
  if (t >= n_q) return;
  const int n_g = (n_q + group - 1) / group;
  const int* src = ptop + ((size_t)b * n_g + t / group) * topk;
  int* dst = out + ((size_t)b * n_q + t) * topk;
  const int pos = q_pos0 + t;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int base = 0;
  for (int c0 = 0; c0 < topk; c0 += kReuseChunks * kWave) {
    int v[kReuseChunks];
#pragma unroll
    for (int j = 0; j < kReuseChunks; ++j) {
      const int c = c0 + j * kWave + lane;
      v[j] = c < topk ? src[c] : -1;
    }
#pragma unroll
    for (int j = 0; j < kReuseChunks; ++j) {
      const bool keep = v[j] >= 0 && v[j] <= pos;
      const unsigned long long m = __ballot(keep);
      if (keep) dst[base + __popcll(m & lt)] = v[j];
      base += __popcll(m);
    }
  }
  for (int i = base + lane; i < topk; i += kWave) dst[i] = -1;
}

hipError_t launch_reuse(const int* ptop, int B, int n_q, int q_pos0, int group, int topk,
                        int* out, hipStream_t st) {
  dim3 grid((n_q + 3) / 4, B);
  hipLaunchKernelGGL(reuse_kernel, grid, dim3(256), 0, st, ptop, n_q, q_pos0, group, topk, out);
  return hipGetLastError();
}

}  // namespace idx
