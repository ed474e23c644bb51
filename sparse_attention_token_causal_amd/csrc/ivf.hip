// IVF candidate routing for gfx950: a clustered index of the keys with causal
// versions, and the routing of group proxies through it.
//
// "AttentionIndex Architecture ...", "KEY FINDINGS" and "An Inverted File
// With Causal Versions": keys are grouped by similarity into inverted lists;
// a query is routed to the lists whose representatives score highest and the
// native indexer re-scores their members.  The index grows with the keys:
// arriving keys join existing lists batch by batch, and from time to time the
// clustering is recomputed over all keys so far, seeded with the last one,
// which yields a new version of lists and representatives.  Causality is kept
// by version: a group may route through version u only when all of u's
// keys precede its last member.  Here the representatives are plain means
// (no trained encoder):
//
//  * version u is refit every R keys on keys [0, u R): T Lloyd iterations of
//    k-means over the stored centroids (bfloat16, float32 for float32 keys),
//    squared-L2 assignment with ties to the lower centroid, the mean of each
//    cluster's members (an empty cluster keeps its centroid), warm-started
//    from version u-1 (version 1 from the keys at positions floor(c R / m));
//  * the published lists of version u hold every key of [0, min((u+1) R, n_k))
//    under its nearest centroid of version u - the refit keys and the keys
//    added in batches until the next refit - ascending within each list,
//    with a table of per-list counts below every 128-key boundary so that a
//    router can cut a list at any batch boundary without searching it.
//
// One Lloyd pass over n keys is three launches: the assignment (MFMA
// distances, 128 keys per workgroup, with each key's rank among its tile's
// keys of the same cluster and per-tile cluster counts), a column scan of
// the counts over tiles, and a stable scatter into the lists.  The mean
// update reads each list in order (fixed summation order: the result does
// not depend on scheduling).  No global atomics anywhere.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <type_traits>

namespace idx {

// Real value of key element (s, e) of sequence b.
template <int KF>
__device__ __forceinline__ float key_real(const void* k, const float* k_scale, int b, int n_k, int D, int s,
                                          int e) {
  const size_t off = ((size_t)b * n_k + s) * D + e;
  if (KF == F32) return ((const float*)k)[off];
  if (KF == BF16) return __uint_as_float((uint32_t)((const uint16_t*)k)[off] << 16);
  return fp8_to_f32(((const uint8_t*)k)[off]) * k_scale[(size_t)b * n_k + s];
}

// Centroids are stored as float32 for float32 keys, bfloat16 otherwise.
template <int KF>
__device__ __forceinline__ void store_cent(void* dst, size_t i, float x) {
  if (KF == F32)
    ((float*)dst)[i] = x;
  else
    ((uint16_t*)dst)[i] = f32_to_bf16_rne(x);
}

template <int KF>
__device__ __forceinline__ float load_cent(const void* src, size_t i) {
  if (KF == F32) return ((const float*)src)[i];
  return __uint_as_float((uint32_t)((const uint16_t*)src)[i] << 16);
}

// ---------------------------------------------------------------------------
// initial centroids of the first version: the keys at positions floor(c R / m)

template <int KF>
__global__ __launch_bounds__(128) void ivf_init_kernel(const void* k, const float* k_scale, int n_k, int D,
                                                       int m, int R, void* dst, long long dst_bs) {
  const int c = blockIdx.x, b = blockIdx.y;
  const int s = (int)((long long)c * R / m);
  for (int e = threadIdx.x; e < D; e += blockDim.x)
    store_cent<KF>(dst, (size_t)b * dst_bs + (size_t)c * D + e, key_real<KF>(k, k_scale, b, n_k, D, s, e));
}

// ---------------------------------------------------------------------------
// assignment: nearest stored centroid of every key of [0, n_assign)
//
// Rows = keys (32 per wave, four waves), columns = centroids staged through
// LDS 64 at a time, contraction over d on MFMA (bfloat16 with FP8 keys
// widened exactly, float32 for float32 keys).  dist = |c|^2 - 2 k.c (|k|^2
// is the same for every centroid); each lane keeps the best of its column
// per row, then a 32-lane reduction takes the smallest distance, ties to the
// lower centroid.

template <int KF, int D>
struct IvfMfma;

template <int D>
struct IvfMfma<F32, D> {
  static constexpr int KSTEP = 2, EB = 4;
  typedef float frag;
  __device__ static frag load_a(const void* k, const float*, int b, int n_k, int s, int ks, int half) {
    return ((const float*)k)[((size_t)b * n_k + s) * D + ks * 2 + half];
  }
  __device__ static frag load_b(const char* row, int ks, int half) {
    return *(const float*)(row + (ks * 2 + half) * 4);
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <int KF, int D>
struct IvfMfmaBf16 {
  static constexpr int KSTEP = 16, EB = 2;
  typedef bf16x8 frag;
  __device__ static frag load_a(const void* k, const float*, int b, int n_k, int s, int ks, int half) {
    const size_t e0 = ((size_t)b * n_k + s) * D + ks * 16 + 8 * half;
    if (KF == BF16) return *(const bf16x8*)((const uint16_t*)k + e0);
    const uint2 codes = *(const uint2*)((const uint8_t*)k + e0);
    uint32_t w0, w1, w2, w3;
    fp8x4_to_bf16x4(codes.x, w0, w1);
    fp8x4_to_bf16x4(codes.y, w2, w3);
    const i32x4 w = {(int)w0, (int)w1, (int)w2, (int)w3};
    return __builtin_bit_cast(bf16x8, w);
  }
  __device__ static frag load_b(const char* row, int ks, int half) {
    return *(const bf16x8*)(row + (ks * 16 + 8 * half) * 2);
  }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <int D>
struct IvfMfma<BF16, D> : IvfMfmaBf16<BF16, D> {};
template <int D>
struct IvfMfma<FP8, D> : IvfMfmaBf16<FP8, D> {};

constexpr int kIvfChunk = 64;  // centroids per LDS chunk of the assignment

template <int KF, int D>
__global__ __launch_bounds__(256) void ivf_assign_kernel(IvfPassArgs a) {
  typedef IvfMfma<KF, D> M;
  constexpr int EB = M::EB, NKS = D / M::KSTEP;
  constexpr int ROWB = D * EB + 16;  // padded LDS row: 16-byte reads of 16 lanes hit distinct banks
  constexpr int CPR = D * EB / 16;   // 16-byte chunks per centroid row
  __shared__ __attribute__((aligned(16))) char s_cent[kIvfChunk * ROWB];
  __shared__ float s_norm[kIvfChunk];
  __shared__ int s_cl[kIvfTile];
  __shared__ int s_cnt[kIvfMaxClusters];

  const int tile = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x / kWave, l = lane_id(), half = l >> 5, l32 = l & 31;
  const int s0 = tile * kIvfTile, m = a.m;
  for (int c = threadIdx.x; c < m; c += blockDim.x) s_cnt[c] = 0;

  // this wave's 32 keys as the A operand (rows past the end repeat the last key)
  const int arow = min(s0 + wave * 32 + l32, a.n_assign - 1);
  typename M::frag af[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) af[ks] = M::load_a(a.k, a.k_scale, b, a.n_k, arow, ks, half);
  float ksc[16], bd[16];
  int bc[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int s = min(s0 + wave * 32 + 8 * (v / 4) + 4 * half + (v % 4), a.n_assign - 1);
    ksc[v] = (KF == FP8) ? a.k_scale[(size_t)b * a.n_k + s] : 1.f;
    bd[v] = __uint_as_float(0x7F800000u);
    bc[v] = 0;
  }

  const char* cbase = (const char*)a.cent + (size_t)b * a.cent_bs * EB;
  for (int c0 = 0; c0 < m; c0 += kIvfChunk) {
    __syncthreads();
    for (int i = threadIdx.x; i < kIvfChunk * CPR; i += blockDim.x) {
      const int r = i / CPR, ch = i % CPR;
      i32x4 v = {0, 0, 0, 0};
      if (c0 + r < m) v = *(const i32x4*)(cbase + (size_t)(c0 + r) * D * EB + ch * 16);
      *(i32x4*)(s_cent + r * ROWB + ch * 16) = v;
    }
    __syncthreads();
    {  // |c|^2 from the stored values: four threads per centroid, fixed order
      const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
      const char* row = s_cent + r * ROWB;
      float acc = 0.f;
      for (int e = part * (D / 4); e < (part + 1) * (D / 4); ++e) {
        const float x = (KF == F32) ? ((const float*)row)[e]
                                    : __uint_as_float((uint32_t)((const uint16_t*)row)[e] << 16);
        acc = fmaf(x, x, acc);
      }
      acc += __shfl_xor(acc, 1, kWave);
      acc += __shfl_xor(acc, 2, kWave);
      if (part == 0) s_norm[r] = (c0 + r < m) ? acc : __uint_as_float(0x7F800000u);
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < kIvfChunk / 32; ++cb) {
      const char* brow = s_cent + (cb * 32 + l32) * ROWB;
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc = M::mma(af[ks], M::load_b(brow, ks, half), acc);
      const float nrm = s_norm[cb * 32 + l32];
      const int c = c0 + cb * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float d = fmaf(-2.f * ksc[v], acc[v], nrm);
        if (d < bd[v]) {
          bd[v] = d;
          bc[v] = c;
        }
      }
    }
  }
  // smallest distance over the 32 columns of each half, ties to the lower centroid
#pragma unroll
  for (int v = 0; v < 16; ++v) {
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float od = __shfl_xor(bd[v], off, kWave);
      const int oc = __shfl_xor(bc[v], off, kWave);
      if (od < bd[v] || (od == bd[v] && oc < bc[v])) {
        bd[v] = od;
        bc[v] = oc;
      }
    }
  }
  if (l32 == 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) s_cl[wave * 32 + 8 * (v / 4) + 4 * half + (v % 4)] = bc[v];
  }
  __syncthreads();
  if (threadIdx.x < kIvfTile) {
    const int i = threadIdx.x, s = s0 + i;
    if (s < a.n_assign) {
      const int c = s_cl[i];
      int r = 0;
      for (int j = 0; j < i; ++j) r += (s_cl[j] == c) ? 1 : 0;
      a.assign[(size_t)b * a.assign_bs + s] = c;
      a.rank[(size_t)b * a.rank_bs + s] = r;
      atomicAdd(&s_cnt[c], 1);
    }
  }
  __syncthreads();
  int* tc = a.tilecnt + (size_t)b * a.tilecnt_bs + (size_t)tile * m;
  for (int c = threadIdx.x; c < m; c += blockDim.x) tc[c] = s_cnt[c];
}

// Column scan of the per-tile counts: counts[t][c] = keys of cluster c in
// tiles before t; row n_tiles holds the cluster totals.  64 clusters per
// workgroup (one per lane), the tiles split over 16 waves.
__global__ __launch_bounds__(1024) void ivf_scan_kernel(IvfPassArgs a, int n_tiles) {
  __shared__ int part[16][64];
  const int b = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane, m = a.m;
  const bool ok = c < m;
  const int tpw = (n_tiles + 15) / 16, t0 = w * tpw, t1 = min(t0 + tpw, n_tiles);
  const int* cnt = a.tilecnt + (size_t)b * a.tilecnt_bs;
  int sum = 0;
  if (ok)
    for (int t = t0; t < t1; ++t) sum += cnt[(size_t)t * m + c];
  part[w][lane] = sum;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int j = 0; j < 16; ++j) {
    const int v = part[j][lane];
    pre += (j < w) ? v : 0;
    tot += v;
  }
  if (!ok) return;
  int* out = a.counts + (size_t)b * a.counts_bs;
  int run = pre;
  for (int t = t0; t < t1; ++t) {
    out[(size_t)t * m + c] = run;
    run += cnt[(size_t)t * m + c];
  }
  if (w == 15) out[(size_t)n_tiles * m + c] = tot;
}

// Exclusive scan of vals[0..n) (n <= 1024) by a 256-thread workgroup into
// dst[0..n]; dst[n] = the total.
__device__ void ivf_block_excl_scan(const int* vals, int n, int* dst, int* wsum) {
  const int per = (n + 255) / 256, tid = threadIdx.x;
  int loc[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid * per + j;
    const int v = (j < per && c < n) ? vals[c] : 0;
    loc[j] = sum;
    sum += v;
  }
  const int incl = wave_incl_scan(sum);
  if (lane_id() == 63) wsum[tid / 64] = incl;
  __syncthreads();
  int base = incl - sum;
  for (int w = 0; w < tid / 64; ++w) base += wsum[w];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid * per + j;
    if (j < per && c < n) dst[c] = base + loc[j];
  }
  if (tid == 0) dst[n] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
}

// Stable scatter into the lists: key s of tile t, cluster c, goes to
// start[c] + counts[t][c] + rank(s).  Workgroup 0 also writes the list offsets.
__global__ __launch_bounds__(256) void ivf_scatter_kernel(IvfPassArgs a, int n_tiles) {
  __shared__ int s_start[kIvfMaxClusters + 1];
  __shared__ int wsum[4];
  const int tile = blockIdx.x, b = blockIdx.y, m = a.m;
  const int* cnt = a.counts + (size_t)b * a.counts_bs;
  ivf_block_excl_scan(cnt + (size_t)n_tiles * m, m, s_start, wsum);
  if (tile == 0) {
    int* off = a.offsets + (size_t)b * a.offsets_bs;
    for (int c = threadIdx.x; c <= m; c += blockDim.x) off[c] = s_start[c];
  }
  const int s = tile * kIvfTile + (int)threadIdx.x;
  if (threadIdx.x < kIvfTile && s < a.n_assign) {
    const int c = a.assign[(size_t)b * a.assign_bs + s];
    const int pos = s_start[c] + cnt[(size_t)tile * m + c] + a.rank[(size_t)b * a.rank_bs + s];
    a.members[(size_t)b * a.members_bs + pos] = s;
  }
}

// ---------------------------------------------------------------------------
// mean update: one workgroup per (cluster, sequence); 512 / D partial sums
// per element over the members in list order (four loads in flight each),
// added in a fixed order.  An empty cluster keeps its centroid.

template <int KF, int D>
__global__ __launch_bounds__(512) void ivf_update_kernel(IvfUpdateArgs a) {
  constexpr int P = 512 / D;
  __shared__ float part[P][D];
  const int c = blockIdx.x, b = blockIdx.y;
  const int p = threadIdx.x / D, e = threadIdx.x % D;
  const int* off = a.offsets + (size_t)b * a.offsets_bs;
  const int start = a.copy_only ? 0 : off[c];
  const int n = a.copy_only ? 0 : off[c + 1] - start;
  const int* mem = a.members + (size_t)b * a.members_bs + start;
  float acc = 0.f;
  int j = p;
  for (; j + 3 * P < n; j += 4 * P) {
    const int s0 = mem[j], s1 = mem[j + P], s2 = mem[j + 2 * P], s3 = mem[j + 3 * P];
    const float x0 = key_real<KF>(a.k, a.k_scale, b, a.n_k, D, s0, e);
    const float x1 = key_real<KF>(a.k, a.k_scale, b, a.n_k, D, s1, e);
    const float x2 = key_real<KF>(a.k, a.k_scale, b, a.n_k, D, s2, e);
    const float x3 = key_real<KF>(a.k, a.k_scale, b, a.n_k, D, s3, e);
    acc += x0;
    acc += x1;
    acc += x2;
    acc += x3;
  }
  for (; j < n; j += P) acc += key_real<KF>(a.k, a.k_scale, b, a.n_k, D, mem[j], e);
  part[p][e] = acc;
  __syncthreads();
  if (p != 0) return;
  const size_t di = (size_t)b * a.dst_bs + (size_t)c * D + e;
  if (n == 0) {
    store_cent<KF>(a.dst, di, load_cent<KF>(a.src, (size_t)b * a.src_bs + (size_t)c * D + e));
    return;
  }
  float t = part[0][e];
#pragma unroll
  for (int q = 1; q < P; ++q) t += part[q][e];
  store_cent<KF>(a.dst, di, t / (float)n);
}

// ---------------------------------------------------------------------------
// routing: cluster scores of each group proxy against its version's centroids

template <int CF, int H, int D>
__global__ __launch_bounds__(256) void ivf_score_kernel(IvfRouteArgs a) {
  typedef IvfMfma<CF == F32 ? F32 : BF16, D> M;
  constexpr int EB = M::EB, NKS = D / M::KSTEP, NRB = (H + 31) / 32;
  const int g = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x / kWave, l = lane_id(), half = l >> 5, l32 = l & 31;
  const int m = a.m;
  float* out = a.scores + ((size_t)b * a.n_g + g) * m;
  const int last = mode_limit(kModeProxy, a.q_pos0, a.n_q, a.group, 1, g);
  const int u = (last + 1) / a.refit;
  if (u == 0) {
    for (int c = threadIdx.x; c < m; c += blockDim.x) out[c] = neg_inf();
    return;
  }
  const char* cent = (const char*)a.cents + ((size_t)b * a.n_v + (u - 1)) * m * D * EB;
  // proxy rows (heads) as the A operand; rows past H are zero with zero weight
  typename M::frag af[NRB][NKS];
  float wreg[NRB][16];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int h = 32 * rb + l32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      typename M::frag f = M::load_a(a.pq, nullptr, 0, 0, (int)(((size_t)b * a.n_g + g) * H + min(h, H - 1)), ks,
                                     half);
      if (h >= H) f = typename M::frag{};
      af[rb][ks] = f;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int hh = 32 * rb + 8 * (v / 4) + 4 * half + (v % 4);
      wreg[rb][v] = hh < H ? a.pw[((size_t)b * a.n_g + g) * H + hh] : 0.f;
    }
  }
  const int n_cb = (m + 31) / 32;
  for (int cb = wave; cb < n_cb; cb += 4) {
    const int c = cb * 32 + l32;
    const char* brow = cent + (size_t)min(c, m - 1) * D * EB;
    float sum = 0.f;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc = M::mma(af[rb][ks], M::load_b(brow, ks, half), acc);
#pragma unroll
      for (int v = 0; v < 16; ++v) sum = fmaf(wreg[rb][v], fmaxf(acc[v], 0.f), sum);
    }
    sum += xor32(sum);
    if (half == 0 && c < m) out[c] = sum;
  }
}

// Expansion of one group's route into its candidate row: clusters in score
// order (descending, ties to the lower index), each taking its members below
// the group's routable end e, while they fit next to the keys [e, last];
// then those keys; then -1.
__global__ __launch_bounds__(256) void ivf_expand_kernel(IvfRouteArgs a) {
  __shared__ float sS[kIvfMaxClusters];
  __shared__ int sOrd[kIvfMaxClusters], sSz[kIvfMaxClusters], sPre[kIvfMaxClusters + 1];
  __shared__ int wsum[4];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, m = a.m;
  const int last = mode_limit(kModeProxy, a.q_pos0, a.n_q, a.group, 1, g);
  const int u = (last + 1) / a.refit;
  int* crow = a.cand + ((size_t)b * a.n_g + g) * a.n_cand;
  if (u == 0) {  // no version yet: the whole prefix
    for (int i = tid; i < a.n_cand; i += blockDim.x) crow[i] = i <= last ? i : -1;
    return;
  }
  const int e = u * a.refit + a.batch * ((last + 1 - u * a.refit) / a.batch);
  const int tail = last + 1 - e;
  const size_t ver = (size_t)b * a.n_v + (u - 1);
  const float* S = a.scores + ((size_t)b * a.n_g + g) * m;
  for (int c = tid; c < m; c += blockDim.x) sS[c] = S[c];
  __syncthreads();
  const int* vis = a.counts + (ver * (a.n_tiles + 1) + e / kIvfTile) * m;
  {  // rank of each cluster in the walk order
    int own[4], r[4];
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      own[j] = tid + 256 * j;
      sv[j] = own[j] < m ? sS[own[j]] : 0.f;
      r[j] = 0;
    }
    for (int c2 = 0; c2 < m; ++c2) {
      const float s2 = sS[c2];
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] += (s2 > sv[j] || (s2 == sv[j] && c2 < own[j])) ? 1 : 0;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (own[j] < m) {
        sOrd[r[j]] = own[j];
        sSz[r[j]] = vis[own[j]];
      }
  }
  __syncthreads();
  ivf_block_excl_scan(sSz, m, sPre, wsum);  // sPre[r] = members of the clusters ranked before r
  const int room = a.n_cand - tail;
  int cnt = 0;
  for (int r = tid; r < m; r += blockDim.x) cnt += (sPre[r + 1] <= room) ? 1 : 0;
  cnt = wave_sum(cnt);
  __syncthreads();
  if (lane_id() == 0) wsum[tid / 64] = cnt;
  __syncthreads();
  const int n_take = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const int P = sPre[n_take];
  const int* off = a.offsets + ver * (m + 1);
  const int* mem = a.members + ver * a.n_k;
  // the taken clusters' list offsets, in walk order (in the sizes' storage:
  // the prefix sums above were their last use, and barriers separate them)
  int* sOff = sSz;
  for (int r = tid; r < n_take; r += 256) sOff[r] = off[sOrd[r]];
  __syncthreads();
  // each thread issues the member loads of eight slots before storing them
  constexpr int XB = 8;
  for (int i0 = 0; i0 < a.n_cand; i0 += XB * 256) {
    int key[XB];
#pragma unroll
    for (int j = 0; j < XB; ++j) {
      const int i = i0 + j * 256 + tid;
      key[j] = -1;
      if (i < P) {
        int lo = 0, hi = n_take - 1;  // last rank r with sPre[r] <= i
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sPre[mid] <= i)
            lo = mid;
          else
            hi = mid - 1;
        }
        key[j] = mem[sOff[lo] + (i - sPre[lo])];
      } else if (i < P + tail) {
        key[j] = e + (i - P);
      }
    }
#pragma unroll
    for (int j = 0; j < XB; ++j) {
      const int i = i0 + j * 256 + tid;
      if (i < a.n_cand) crow[i] = key[j];
    }
  }
}

__global__ void fill_i32_kernel(int* p, size_t n, int v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---------------------------------------------------------------------------
// launchers

hipError_t launch_fill_i32(int* p, size_t n, int v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_ivf_init(const void* k, const float* k_scale, int kf, int B, int n_k, int D, int m, int R,
                           void* dst, long long dst_bs, hipStream_t st) {
  dim3 grid(m, B);
  if (kf == F32)
    hipLaunchKernelGGL(ivf_init_kernel<F32>, grid, dim3(128), 0, st, k, k_scale, n_k, D, m, R, dst, dst_bs);
  else if (kf == BF16)
    hipLaunchKernelGGL(ivf_init_kernel<BF16>, grid, dim3(128), 0, st, k, k_scale, n_k, D, m, R, dst, dst_bs);
  else
    hipLaunchKernelGGL(ivf_init_kernel<FP8>, grid, dim3(128), 0, st, k, k_scale, n_k, D, m, R, dst, dst_bs);
  return hipGetLastError();
}

template <int KF, int D>
static void assign_kd(const IvfPassArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((ivf_assign_kernel<KF, D>), grid, dim3(256), 0, st, a);
}

hipError_t launch_ivf_pass(const IvfPassArgs& a, int kf, int D, int B, hipStream_t st) {
  const int n_tiles = (a.n_assign + kIvfTile - 1) / kIvfTile;
  const dim3 grid(n_tiles, B);
  if (D == 64) {
    if (kf == F32) assign_kd<F32, 64>(a, grid, st);
    else if (kf == BF16) assign_kd<BF16, 64>(a, grid, st);
    else assign_kd<FP8, 64>(a, grid, st);
  } else {
    if (kf == F32) assign_kd<F32, 128>(a, grid, st);
    else if (kf == BF16) assign_kd<BF16, 128>(a, grid, st);
    else assign_kd<FP8, 128>(a, grid, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ivf_scan_kernel, dim3((a.m + 63) / 64, B), dim3(1024), 0, st, a, n_tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ivf_scatter_kernel, grid, dim3(256), 0, st, a, n_tiles);
  return hipGetLastError();
}

template <int KF, int D>
static void update_kd(const IvfUpdateArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((ivf_update_kernel<KF, D>), grid, dim3(512), 0, st, a);
}

hipError_t launch_ivf_update(const IvfUpdateArgs& a, int kf, int D, int B, hipStream_t st) {
  const dim3 grid(a.m, B);
  if (D == 64) {
    if (kf == F32) update_kd<F32, 64>(a, grid, st);
    else if (kf == BF16) update_kd<BF16, 64>(a, grid, st);
    else update_kd<FP8, 64>(a, grid, st);
  } else {
    if (kf == F32) update_kd<F32, 128>(a, grid, st);
    else if (kf == BF16) update_kd<BF16, 128>(a, grid, st);
    else update_kd<FP8, 128>(a, grid, st);
  }
  return hipGetLastError();
}

template <int CF, int H, int D>
static void score_chd(const IvfRouteArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((ivf_score_kernel<CF, H, D>), grid, dim3(256), 0, st, a);
}

template <int CF, int H>
static void score_ch(const IvfRouteArgs& a, int D, dim3 grid, hipStream_t st) {
  if (D == 64) score_chd<CF, H, 64>(a, grid, st);
  else score_chd<CF, H, 128>(a, grid, st);
}

template <int CF>
static void score_c(const IvfRouteArgs& a, int H, int D, dim3 grid, hipStream_t st) {
  if (H == 16) score_ch<CF, 16>(a, D, grid, st);
  else if (H == 32) score_ch<CF, 32>(a, D, grid, st);
  else score_ch<CF, 64>(a, D, grid, st);
}

hipError_t launch_ivf_route(const IvfRouteArgs& a, int cf, int H, int D, int B, hipStream_t st) {
  const dim3 grid(a.n_g, B);
  if (cf == F32) score_c<F32>(a, H, D, grid, st);
  else score_c<BF16>(a, H, D, grid, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ivf_expand_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace idx
