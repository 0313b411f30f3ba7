// Cluster-granularity recall (ClusterKV article, "大模型KV Cache压缩技术：
// ClusterKV的语义空间优化", §3.3; §3.1 motivates ranking clusters by q.mu).
//
// Per unit (one KV head of one sequence): q_bar = sum of the group's query
// heads; cluster score s_j = q_bar . mu_j (-inf for an empty cluster);
// clusters in descending score (ties: smaller j) are taken whole while they
// fit; the first that does not fit contributes its highest q_bar.k tokens
// (ties: smaller position) so exactly min(budget, m) tokens are recalled.
//
// Two kernels: a wide scoring pass (16 lanes per centroid row, many
// workgroups per unit) and one workgroup per unit for rank, prefix sum, cut
// and a 4-pass radix select inside the cut cluster.
#include "common.hpp"
#include "launch.hpp"

namespace ckv {

constexpr int kScorePerWg = 64;

__global__ __launch_bounds__(256) void select_score_kernel(const uint16_t* __restrict__ q, int G,
                                                           const float* __restrict__ cmean,
                                                           const int32_t* __restrict__ offsets,
                                                           int K, float* __restrict__ scores,
                                                           int tiles) {
  const int u = blockIdx.x / tiles;
  const int t = blockIdx.x % tiles;
  const int li = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  float qb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qb[e] = 0.f;
  for (int h = 0; h < G; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(q + ((size_t)u * G + h) * kHeadDim + li * 8);
    qb[0] += bf16_lo(w.x); qb[1] += bf16_hi(w.x);
    qb[2] += bf16_lo(w.y); qb[3] += bf16_hi(w.y);
    qb[4] += bf16_lo(w.z); qb[5] += bf16_hi(w.z);
    qb[6] += bf16_lo(w.w); qb[7] += bf16_hi(w.w);
  }
  for (int jj = grp; jj < kScorePerWg; jj += 16) {
    const int j = t * kScorePerWg + jj;
    if (j >= K) break;
    const float* mp = cmean + ((size_t)u * K + j) * kHeadDim + li * 8;
    const float4 m0 = *reinterpret_cast<const float4*>(mp);
    const float4 m1 = *reinterpret_cast<const float4*>(mp + 4);
    float d = qb[0] * m0.x;
    d = fmaf(qb[1], m0.y, d); d = fmaf(qb[2], m0.z, d); d = fmaf(qb[3], m0.w, d);
    d = fmaf(qb[4], m1.x, d); d = fmaf(qb[5], m1.y, d); d = fmaf(qb[6], m1.z, d);
    d = fmaf(qb[7], m1.w, d);
    d = xor_sum16(d);
    if (li == 0) {
      const int n = offsets[(size_t)u * (K + 1) + j + 1] - offsets[(size_t)u * (K + 1) + j];
      scores[(size_t)u * K + j] = n > 0 ? d : -INFINITY;
    }
  }
}

// Order-preserving map of an f32 score to u32 (larger score -> larger key); -0 maps as +0.
__device__ __forceinline__ uint32_t score_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Block-wide exclusive scan over arbitrary length arrays processed in chunks
// of blockDim.x; `running` carries the sum of earlier chunks.
__global__ __launch_bounds__(256) void select_finish_kernel(
    const uint16_t* __restrict__ q, int G, const float* __restrict__ scores,
    const int32_t* __restrict__ offsets, int K, const uint16_t* __restrict__ k_clu,
    int clu_stride, int budget, int32_t* __restrict__ sel_pos, int32_t* __restrict__ sel_count,
    uint32_t* __restrict__ cut_ws) {
  __shared__ float sc[kMaxClusters];
  __shared__ int sz[kMaxClusters];
  __shared__ int rk[kMaxClusters];
  __shared__ int pre[kMaxClusters];
  __shared__ int ost[kMaxClusters];
  __shared__ int hist[256];
  __shared__ int scan_scratch[8];
  __shared__ int sh_rcut, sh_jcut, sh_need, sh_prefix, sh_rem;

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int32_t* off = offsets + (size_t)u * (K + 1);
  const int m = off[K];
  const int beff = budget < m ? budget : m;

  for (int j = tid; j < K; j += blockDim.x) {
    sc[j] = scores[(size_t)u * K + j];
    sz[j] = off[j + 1] - off[j];
  }
  if (tid == 0) {
    sh_rcut = K;
    sh_jcut = -1;
  }
  __syncthreads();
  // rank_j = #{i : s_i > s_j or (s_i == s_j and i < j)}
  for (int j = tid; j < K; j += blockDim.x) {
    const float s = sc[j];
    int r = 0;
    for (int i = 0; i < K; ++i) {
      const float si = sc[i];
      r += (si > s) || (si == s && i < j);
    }
    rk[j] = r;
  }
  __syncthreads();
  for (int j = tid; j < K; j += blockDim.x) pre[rk[j]] = sz[j];
  __syncthreads();
  // inclusive prefix over ranks
  {
    int running = 0;
    for (int c0 = 0; c0 < K; c0 += blockDim.x) {
      const int r = c0 + tid;
      const int v = r < K ? pre[r] : 0;
      int tot;
      const int ex = block_exclusive_scan(v, scan_scratch, &tot);
      if (r < K) pre[r] = running + ex + v;
      running += tot;
    }
  }
  __syncthreads();
  for (int r = tid; r < K; r += blockDim.x) {
    const int below = r == 0 ? 0 : pre[r - 1];
    if (pre[r] > beff && below <= beff) {
      sh_rcut = r;
      sh_need = beff - below;
    }
  }
  __syncthreads();
  const int rcut = sh_rcut;
  for (int j = tid; j < K; j += blockDim.x)
    if (rk[j] == rcut) sh_jcut = j;
  __syncthreads();
  const int jcut = rcut < K ? sh_jcut : -1;
  const int need = rcut < K ? sh_need : 0;
  // output start of every cluster in index (= position) order
  {
    int running = 0;
    for (int c0 = 0; c0 < K; c0 += blockDim.x) {
      const int j = c0 + tid;
      int take = 0;
      if (j < K) take = rk[j] < rcut ? sz[j] : (j == jcut ? need : 0);
      int tot;
      const int ex = block_exclusive_scan(take, scan_scratch, &tot);
      if (j < K) ost[j] = running + ex;
      running += tot;
    }
  }
  __syncthreads();
  int32_t* out = sel_pos + (size_t)u * budget;
  for (int j = wave; j < K; j += blockDim.x / kWave) {
    if (rk[j] < rcut) {
      const int lo = off[j], o = ost[j], n = sz[j];
      for (int t = lane; t < n; t += kWave) out[o + t] = lo + t;
    }
  }

  if (jcut >= 0 && need > 0) {
    const int lo = off[jcut];
    const int n = sz[jcut];
    uint32_t* keys = cut_ws + (size_t)u * clu_stride;
    // scores of the cut cluster's tokens: 16 lanes per row
    const int li = tid & 15, grp = tid >> 4;
    float qb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[e] = 0.f;
    for (int h = 0; h < G; ++h) {
      const uint4 w = *reinterpret_cast<const uint4*>(q + ((size_t)u * G + h) * kHeadDim + li * 8);
      qb[0] += bf16_lo(w.x); qb[1] += bf16_hi(w.x);
      qb[2] += bf16_lo(w.y); qb[3] += bf16_hi(w.y);
      qb[4] += bf16_lo(w.z); qb[5] += bf16_hi(w.z);
      qb[6] += bf16_lo(w.w); qb[7] += bf16_hi(w.w);
    }
    for (int i = grp; i < n; i += blockDim.x / 16) {
      const uint4 w = *reinterpret_cast<const uint4*>(k_clu + ((size_t)u * clu_stride + lo + i) * kHeadDim + li * 8);
      float d = qb[0] * bf16_lo(w.x);
      d = fmaf(qb[1], bf16_hi(w.x), d); d = fmaf(qb[2], bf16_lo(w.y), d);
      d = fmaf(qb[3], bf16_hi(w.y), d); d = fmaf(qb[4], bf16_lo(w.z), d);
      d = fmaf(qb[5], bf16_hi(w.z), d); d = fmaf(qb[6], bf16_lo(w.w), d);
      d = fmaf(qb[7], bf16_hi(w.w), d);
      d = xor_sum16(d);
      if (li == 0) keys[i] = score_key(d);
    }
    if (tid == 0) {
      sh_prefix = 0;
      sh_rem = need;
    }
    __syncthreads();
    // radix select of the need-th largest key, 8 bits per pass from the top
    uint32_t mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      const uint32_t prefix = (uint32_t)sh_prefix;
      for (int i = tid; i < n; i += blockDim.x) {
        const uint32_t k = keys[i];
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int rem = sh_rem, cum = 0;
        for (int b = 255; b >= 0; --b) {
          if (cum + hist[b] >= rem) {
            sh_prefix = (int)(prefix | ((uint32_t)b << shift));
            sh_rem = rem - cum;
            break;
          }
          cum += hist[b];
        }
      }
      mask |= 255u << shift;
      __syncthreads();
    }
    const uint32_t T = (uint32_t)sh_prefix;
    const int rem_eq = sh_rem;  // how many of the key == T tokens to take (smallest positions)
    int run_eq = 0, run_sel = 0;
    const int o = ost[jcut];
    for (int c0 = 0; c0 < n; c0 += blockDim.x) {
      const int i = c0 + tid;
      const uint32_t k = i < n ? keys[i] : 0u;
      const int eq = (i < n && k == T) ? 1 : 0;
      int tot_eq;
      const int ex_eq = block_exclusive_scan(eq, scan_scratch, &tot_eq);
      const int sel = (i < n) && (k > T || (eq && run_eq + ex_eq < rem_eq)) ? 1 : 0;
      int tot_sel;
      const int ex_sel = block_exclusive_scan(sel, scan_scratch, &tot_sel);
      if (sel) out[o + run_sel + ex_sel] = lo + i;
      run_eq += tot_eq;
      run_sel += tot_sel;
    }
  }
  if (tid == 0) sel_count[u] = beff;
}

hipError_t launch_select(const uint16_t* q, int group, const float* cmean, const int32_t* offsets,
                         int K, const uint16_t* k_clu, int clu_stride, int budget, int32_t* sel_pos,
                         int32_t* sel_count, float* scores_ws, uint32_t* cut_ws, int units,
                         hipStream_t s) {
  const int tiles = (K + kScorePerWg - 1) / kScorePerWg;
  hipLaunchKernelGGL(select_score_kernel, dim3((unsigned)(units * tiles)), dim3(256), 0, s, q, group,
                     cmean, offsets, K, scores_ws, tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_finish_kernel, dim3((unsigned)units), dim3(256), 0, s, q, group,
                     scores_ws, offsets, K, k_clu, clu_stride, budget, sel_pos, sel_count, cut_ws);
  return hipGetLastError();
}

}  // namespace ckv
