// Cluster-granularity recall (ClusterKV article, "大模型KV Cache压缩技术：
// ClusterKV的语义空间优化", §3.3; §3.1 motivates ranking clusters by q.mu).
//
// Per unit (one KV head of one sequence): q_bar = sum of the group's query
// heads; cluster score s_j = q_bar . mu_j (an empty cluster never scores);
// clusters in descending score (ties: smaller j) are taken whole while they
// fit; the first that does not fit contributes its highest q_bar.k tokens
// (ties: smaller position) so exactly min(budget, m) tokens are recalled.
//
// The walk in score order is a weighted selection: the cut cluster is the one
// whose score key T splits the clusters into those above T (taken whole,
// total size <= budget) and the rest.  It is found without sorting by a
// wave-synchronous radix select on order-preserving 32-bit score keys with
// cluster sizes as weights (4 passes of 8 bits); the partial fill inside the
// cut cluster is the same select with unit weights.  One workgroup of 1024
// threads per unit, three block barriers; recalled positions are written by
// whole waves so every store instruction covers 64 consecutive slots.
#include "common.hpp"
#include "launch.hpp"

namespace ckv {

constexpr int kSelThreads = 1024;
constexpr int kSelGroups = kSelThreads / 16;  // 16-lane row groups
constexpr int kCutLds = 4096;                 // cut-cluster keys kept in LDS up to this size

// Order-preserving map of an f32 score to u32 (larger score -> larger key);
// -0 maps as +0.  Every finite or infinite score maps above 0, which is kept
// for empty clusters.
__device__ __forceinline__ uint32_t score_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

constexpr int kRegKeys = 16;
constexpr int kHistBins = 256 + 4;  // one dummy bin (index 256) takes keys outside the prefix
constexpr int kHistCopies = 8;      // lane % 8 picks a copy: same-bin LDS atomics conflict 8x less

// Pick the digit bin where the descending running weight crosses `rem`.
// Lane l owns bins 255-4l .. 252-4l (one 16-byte LDS load per histogram copy).
__device__ __forceinline__ int radix_pick_bin(const int* hist, int rem, int* above_out) {
  const int lane = lane_id();
  int4 hb = make_int4(0, 0, 0, 0);
#pragma unroll
  for (int c = 0; c < kHistCopies; ++c) {
    const int4 v = *reinterpret_cast<const int4*>(hist + c * kHistBins + 252 - 4 * lane);
    hb.x += v.x; hb.y += v.y; hb.z += v.z; hb.w += v.w;
  }
  const int h0 = hb.w, h1 = hb.z, h2 = hb.y, h3 = hb.x;
  const int tot = h0 + h1 + h2 + h3;
  const int c0 = wave_incl_scan(tot) - tot;
  const int c1 = c0 + h0, c2 = c1 + h1, c3 = c2 + h2, c4 = c3 + h3;
  const bool in = c0 <= rem && rem < c4;
  const int sub = rem < c1 ? 0 : (rem < c2 ? 1 : (rem < c3 ? 2 : 3));
  const int above = sub == 0 ? c0 : (sub == 1 ? c1 : (sub == 2 ? c2 : c3));
  const unsigned long long bal = __ballot(in);
  const int src = bal ? (int)__ffsll((long long)bal) - 1 : 0;
  *above_out = __builtin_amdgcn_readlane(above, src);
  const int bsel = 255 - 4 * src - __builtin_amdgcn_readlane(sub, src);
  return bal ? bsel : 0;  // no bin only if the precondition fails; keeps the result defined
}

// Wave-synchronous weighted radix select over n keys (descending).
// Precondition: the total weight exceeds `rem`.  Returns the key T of the
// element at which the running weight (in descending key order) first
// exceeds `rem`, and rem minus the weight of all keys above T.  Zero-weight
// keys never count.  CACHED: n <= 64 * kRegKeys, keys and weights held in
// registers; otherwise they are re-read from memory every pass.  The leading
// bits every counted key shares are skipped (often only 2-3 passes of 8 bits).
template <bool CACHED>
__device__ __forceinline__ void wave_radix_select(const uint32_t* keys, const int* weights, int n, int rem,
                                                  int* hist, uint32_t* T_out, int* rem_out) {
  const int lane = lane_id();
  const int live = (n + kWave - 1) / kWave;
  uint32_t rk[CACHED ? kRegKeys : 1];
  int rw[CACHED ? kRegKeys : 1];
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
  if (CACHED) {
#pragma unroll
    for (int t = 0; t < kRegKeys; ++t) {
      const int i = lane + t * kWave;
      // keys / weights arrays hold at least 64 * kRegKeys entries: read unconditionally
      const bool ok = t < live && i < n;
      const uint32_t kv = keys[i];
      const int wv = weights ? weights[i] : 1;
      rk[t] = ok ? kv : 0u;
      rw[t] = ok ? wv : 0;
      kand &= rw[t] > 0 ? rk[t] : 0xFFFFFFFFu;
      kor |= rw[t] > 0 ? rk[t] : 0u;
    }
  } else {
    for (int i = lane; i < n; i += kWave) {
      if ((weights ? weights[i] : 1) > 0) {
        kand &= keys[i];
        kor |= keys[i];
      }
    }
  }
  kand = wave_and(kand);
  kor = wave_or(kor);
  const uint32_t diff = kand ^ kor;
  if (!diff) {  // every counted key is equal
    *T_out = kand;
    *rem_out = rem;
    return;
  }
  const int top = (31 - __clz((int)diff)) >> 3;  // byte holding the highest differing bit
  uint32_t mask = top == 3 ? 0u : (0xFFFFFFFFu << (8 * (top + 1)));
  uint32_t prefix = kand & mask;
  for (int shift = 8 * top; shift >= 0; shift -= 8) {
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c)
      *reinterpret_cast<int4*>(hist + c * kHistBins + 4 * lane) = make_int4(0, 0, 0, 0);
    int* hc = hist + (lane % kHistCopies) * kHistBins;
    if (CACHED) {
#pragma unroll
      for (int t = 0; t < kRegKeys; ++t) {
        if (t >= live) break;
        const bool in = rw[t] > 0 && (rk[t] & mask) == prefix;
        atomicAdd(&hc[in ? (int)((rk[t] >> shift) & 255) : 256], rw[t]);
      }
    } else {
      for (int i = lane; i < n; i += kWave) {
        const uint32_t k = keys[i];
        const int w = weights ? weights[i] : 1;
        const bool in = w > 0 && (k & mask) == prefix;
        atomicAdd(&hc[in ? (int)((k >> shift) & 255) : 256], w);
      }
    }
    int above;
    const int bsel = radix_pick_bin(hist, rem, &above);
    prefix |= (uint32_t)bsel << shift;
    mask |= 255u << shift;
    rem -= above;
  }
  *T_out = prefix;
  *rem_out = rem;
}

__device__ __forceinline__ void qbar8(const uint16_t* q, int u, int G, int li, float* qb) {
#pragma unroll
  for (int e = 0; e < 8; ++e) qb[e] = 0.f;
  for (int h = 0; h < G; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(q + ((size_t)u * G + h) * kHeadDim + li * 8);
    qb[0] += bf16_lo(w.x); qb[1] += bf16_hi(w.x);
    qb[2] += bf16_lo(w.y); qb[3] += bf16_hi(w.y);
    qb[4] += bf16_lo(w.z); qb[5] += bf16_hi(w.z);
    qb[6] += bf16_lo(w.w); qb[7] += bf16_hi(w.w);
  }
}

// Partial fill of the cut cluster by one wave: the `need` highest token keys
// (ties: smaller position first), written in position order at `o`.
__device__ __forceinline__ void fill_cut(const uint32_t* tk, int n, int need, int lo, int o, int* hist,
                                         int32_t* out) {
  const int lane = lane_id();
  uint32_t T2;
  int rem2;
  if (n <= kWave * kRegKeys)
    wave_radix_select<true>(tk, nullptr, n, need, hist, &T2, &rem2);
  else
    wave_radix_select<false>(tk, nullptr, n, need, hist, &T2, &rem2);
  // rem2 = how many of the key == T2 tokens to take, smallest positions first
  int run_eq = 0, run_sel = 0;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + lane;
    const uint32_t k = i < n ? tk[i] : 0u;
    const int eq = (i < n && k == T2) ? 1 : 0;
    const int eq_incl = wave_incl_scan(eq);
    const bool sel = i < n && (k > T2 || (eq && run_eq + eq_incl - 1 < rem2));
    const unsigned long long sb = __ballot(sel);
    if (sel) out[o + run_sel + __popcll(sb & lt)] = lo + i;
    run_sel += __popcll(sb);
    run_eq += __builtin_amdgcn_readlane(eq_incl, kWave - 1);
  }
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const uint16_t* __restrict__ q, int G, const float* __restrict__ cmean,
    const int32_t* __restrict__ offsets, int K, const uint16_t* __restrict__ k_clu, int clu_stride,
    int budget, int32_t* __restrict__ sel_pos, int32_t* __restrict__ sel_count,
    uint32_t* __restrict__ cut_ws) {
  __shared__ uint32_t key[kMaxClusters];
  __shared__ int sz[kMaxClusters];
  __shared__ int ost[kMaxClusters + 1];
  __shared__ int take[kMaxClusters];
  __shared__ __attribute__((aligned(16))) int hist[kHistCopies * kHistBins];
  __shared__ uint32_t tkey[kCutLds];
  __shared__ int sh_cut, sh_need;
  __shared__ uint32_t sh_T;

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int li = tid & 15;
  const int grp = tid >> 4;
  const int32_t* off = offsets + (size_t)u * (K + 1);
  const int m = off[K];
  const int beff = budget < m ? budget : m;

  float qb[8];
  qbar8(q, u, G, li, qb);

  // ---- cluster score keys: 16 lanes per centroid row, 8 rows in flight per group
  constexpr int kRowsInFlight = 8;
  const float* mu_u = cmean + (size_t)u * K * kHeadDim + li * 8;
  for (int j0 = grp; j0 < K; j0 += kSelGroups * kRowsInFlight) {
    float4 a[kRowsInFlight][2];
    int nsz[kRowsInFlight];
#pragma unroll
    for (int t = 0; t < kRowsInFlight; ++t) {
      const int j = j0 + t * kSelGroups;
      const int jc = j < K ? j : K - 1;
      nsz[t] = off[jc + 1] - off[jc];
      if (j < K) {
        a[t][0] = *reinterpret_cast<const float4*>(mu_u + (size_t)j * kHeadDim);
        a[t][1] = *reinterpret_cast<const float4*>(mu_u + (size_t)j * kHeadDim + 4);
      } else {
        a[t][0] = a[t][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int t = 0; t < kRowsInFlight; ++t) {
      const int j = j0 + t * kSelGroups;
      float d = qb[0] * a[t][0].x;
      d = fmaf(qb[1], a[t][0].y, d); d = fmaf(qb[2], a[t][0].z, d); d = fmaf(qb[3], a[t][0].w, d);
      d = fmaf(qb[4], a[t][1].x, d); d = fmaf(qb[5], a[t][1].y, d); d = fmaf(qb[6], a[t][1].z, d);
      d = fmaf(qb[7], a[t][1].w, d);
      d = sum16(d);
      if (li == 0 && j < K) {
        sz[j] = nsz[t];
        key[j] = nsz[t] > 0 ? score_key(d) : 0u;  // empty clusters rank below every score
      }
    }
  }
  __syncthreads();

  // ---- phase 2, wave 0: the cut cluster (weighted radix select on the score keys)
  if (wave == 0) {
    int cut = -1, need = 0;
    uint32_t T = 0;
    if (m > budget) {
      int rem;
      wave_radix_select<true>(key, sz, K, beff, hist, &T, &rem);
      // clusters with key == T are visited in index order: the cut is the first
      // whose running size exceeds what is left
      int run = 0;
      for (int j0 = 0; j0 < K; j0 += kWave) {
        const int j = j0 + lane;
        const bool eq = j < K && key[j] == T;
        const int w = eq ? sz[j] : 0;
        const int incl = run + wave_incl_scan(w);
        const bool hit = eq && incl > rem && incl - w <= rem;
        const unsigned long long b = __ballot(hit);
        if (b) {
          const int src = (int)__ffsll((long long)b) - 1;
          cut = __builtin_amdgcn_readlane(j, src);
          need = rem - __builtin_amdgcn_readlane(incl - w, src);
          break;
        }
        run = __builtin_amdgcn_readlane(incl, kWave - 1);
      }
    }
    if (lane == 0) {
      sh_cut = cut;
      sh_need = need;
      sh_T = T;
    }
  }
  __syncthreads();
  const int cut = sh_cut;
  const int need = sh_need;
  const int n_cut = cut >= 0 ? sz[cut] : 0;
  const int lo_cut = cut >= 0 ? off[cut] : 0;
  const bool fill = cut >= 0 && need > 0;
  uint32_t* cut_keys_g = cut_ws + (size_t)u * clu_stride;

  // ---- phase 3: waves 1.. score the cut cluster's tokens while wave 0 lays out
  // the output (take_j and its exclusive scan over clusters in index order)
  if (wave == 0) {
    const uint32_t T = sh_T;
    int run = 0;
    for (int j0 = 0; j0 < K; j0 += kWave) {
      const int j = j0 + lane;
      int t = 0;
      if (j < K) {
        if (cut < 0) {
          t = sz[j];
        } else {
          const uint32_t k = key[j];
          t = (k > T || (k == T && j < cut)) ? sz[j] : (j == cut ? need : 0);
        }
      }
      const int incl = wave_incl_scan(t);
      if (j < K) {
        ost[j] = run + incl - t;
        take[j] = t;
      }
      run += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
  } else if (fill) {
    constexpr int kGroups = kSelGroups - kWave / 16;  // row groups outside wave 0
    const int g = grp - kWave / 16;
    const uint16_t* kc = k_clu + ((size_t)u * clu_stride + lo_cut) * kHeadDim + li * 8;
    for (int i0 = g; i0 < n_cut; i0 += kGroups * 4) {
      uint4 w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = i0 + t * kGroups;
        w[t] = i < n_cut ? *reinterpret_cast<const uint4*>(kc + (size_t)i * kHeadDim) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = i0 + t * kGroups;
        float d = qb[0] * bf16_lo(w[t].x);
        d = fmaf(qb[1], bf16_hi(w[t].x), d); d = fmaf(qb[2], bf16_lo(w[t].y), d);
        d = fmaf(qb[3], bf16_hi(w[t].y), d); d = fmaf(qb[4], bf16_lo(w[t].z), d);
        d = fmaf(qb[5], bf16_hi(w[t].z), d); d = fmaf(qb[6], bf16_lo(w[t].w), d);
        d = fmaf(qb[7], bf16_hi(w[t].w), d);
        d = sum16(d);
        if (li == 0 && i < n_cut) {
          if (n_cut <= kCutLds)
            tkey[i] = score_key(d);
          else
            cut_keys_g[i] = score_key(d);
        }
      }
    }
  }
  __syncthreads();

  // ---- phase 4: waves 1.. write whole clusters (positions off_j .. off_j + n_j - 1
  // at ost_j, 64 slots per store instruction); wave 0 fills the cut cluster
  int32_t* out = sel_pos + (size_t)u * budget;
  if (wave != 0) {
    constexpr int kWriters = kSelThreads / kWave - 1;
    for (int jb = (wave - 1) * kWave; jb < K; jb += kWriters * kWave) {
      const int j = jb + lane;
      const int t = (j < K && j != cut) ? take[j] : 0;
      const int o = j < K ? ost[j] : 0;
      const int lo = j < K ? off[j] : 0;
      unsigned long long live = __ballot(t > 0);
      while (live) {
        const int l = (int)__ffsll((long long)live) - 1;
        live &= live - 1;
        const int tl = __builtin_amdgcn_readlane(t, l), ol = __builtin_amdgcn_readlane(o, l);
        const int ll = __builtin_amdgcn_readlane(lo, l);
        for (int i = lane; i < tl; i += kWave) out[ol + i] = ll + i;
      }
    }
  } else if (fill) {
    if (n_cut <= kCutLds)
      fill_cut(tkey, n_cut, need, lo_cut, ost[cut], hist, out);
    else
      fill_cut(cut_keys_g, n_cut, need, lo_cut, ost[cut], hist, out);
  }
  if (tid == 0) sel_count[u] = beff;
}

hipError_t launch_select(const uint16_t* q, int group, const float* cmean, const int32_t* offsets,
                         int K, const uint16_t* k_clu, int clu_stride, int budget, int32_t* sel_pos,
                         int32_t* sel_count, float* scores_ws, uint32_t* cut_ws, int units,
                         hipStream_t s) {
  (void)scores_ws;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)units), dim3(kSelThreads), 0, s, q, group, cmean,
                     offsets, K, k_clu, clu_stride, budget, sel_pos, sel_count, cut_ws);
  return hipGetLastError();
}

}  // namespace ckv
