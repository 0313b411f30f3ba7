// Cluster-granularity recall (ClusterKV article, "大模型KV Cache压缩技术：
// ClusterKV的语义空间优化", §3.3; §3.1 motivates ranking clusters by q.mu).
//
// Per unit (one KV head of one sequence): q_bar = sum of the group's query
// heads; cluster score s_j = q_bar . mu_j (an empty cluster never scores);
// clusters in descending score (ties: smaller j) are taken whole while they
// fit; the first that does not fit contributes its highest q_bar.k tokens
// (ties: smaller position) so exactly min(budget, m) tokens are recalled.
//
// The selection itself (bucketed weighted select, no sort) is in recall.hpp.
// Several workgroups of 1024 threads per recalled set (4 up to 64 sets, then
// about 256 per launch, never fewer than K / 256) each score a share of the
// clusters; the last of them to finish (device-scope arrival counter) makes
// the selection.
// A set is one KV head's recall (q_bar over its G query heads) or, in the
// per-query-head mode, one query head's (q_g alone).  The barriers wait on LDS
// only, so global loads stay in flight across them.  Recalled positions are
// written by whole waves, 64 consecutive slots per store instruction.
#include "recall.hpp"

namespace ckv {

constexpr int kSelThreads = 1024;
// Workgroups per recalled set for the cluster scores: about 256 scoring
// workgroups per launch (one per CU) when there are fewer sets, at least
// enough to cover K with one round of row loads per workgroup, at most
// kSelSplitMax (8 per set measured slower than 4 at 32 sets: the hand-off
// waits for more arrivals).
constexpr int kSelSplitMax = 4;
constexpr int kSelRowsPerWg = 256;  // cluster rows one scoring workgroup covers
constexpr int kSelGroups = kSelThreads / 16;  // 16-lane row groups
constexpr int kSelWaves = kSelThreads / kWave;

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const uint16_t* __restrict__ q, int G, const float* __restrict__ cmean,
    const int32_t* __restrict__ offsets, int K, const uint16_t* __restrict__ k_clu, int clu_stride,
    int budget, int32_t* __restrict__ sel_pos, int32_t* __restrict__ sel_count, float* __restrict__ scores_ws,
    uint32_t* __restrict__ cut_ws, uint32_t* __restrict__ counters, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_tok, uint16_t* __restrict__ v_tok, int capacity,
    int row, int hs, int nsplit) {
  __shared__ __attribute__((aligned(16))) uint32_t key[kMaxClusters];
  __shared__ __attribute__((aligned(16))) float csc[kMaxClusters];
  __shared__ __attribute__((aligned(16))) int sz[kMaxClusters];
  __shared__ int ost[kMaxClusters];
  __shared__ int take[kMaxClusters];
  __shared__ __attribute__((aligned(16))) int hist[kHistCopies * kHistBins];
  __shared__ __attribute__((aligned(16))) uint32_t tkey[kCutLds];
  __shared__ __attribute__((aligned(16))) float tsc[kCutLds];
  __shared__ __attribute__((aligned(16))) SelScratch<kSelThreads> ws;
  __shared__ int sh_last;
  __shared__ __attribute__((aligned(16))) float qbar_lds[kHeadDim];  // the group's query sum

  // selection v of physical unit u: hs = 1 (one recall per KV head, q_bar over
  // its G query heads) or hs = G (one recall per query head, G passed as 1)
  const int v = blockIdx.x / nsplit;
  const int u = v / hs;
  const int part = blockIdx.x % nsplit;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int li = tid & 15;
  const int grp = tid >> 4;
  const int32_t* off = offsets + (size_t)u * (K + 1);
  const int m = off[K];
  const int beff = budget < m ? budget : m;

  // fused append of the decoded token's K and V rows (row `row` of the
  // token-order cache, which recall never reads)
  if (k_new != nullptr && part == 0 && tid < 32) {
    const int c8 = (tid & 15) * 8;
    const uint16_t* src = (tid < 16 ? k_new : v_new) + (size_t)u * kHeadDim + c8;
    uint16_t* dst = (tid < 16 ? k_tok : v_tok) + ((size_t)u * capacity + row) * kHeadDim + c8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }

  // ---- phase 1: this workgroup's share of the cluster scores (16 lanes per
  // centroid row, every row of the share in flight at once), stored
  // device-scope; the last workgroup of the unit to finish goes on
  constexpr int kRowsInFlight = 4;
  static_assert(kSelGroups * kRowsInFlight == kSelRowsPerWg, "one round of row loads covers the share");
  const int j_lo = part * K / nsplit, j_hi = (part + 1) * K / nsplit;
  const float* mu_u = cmean + (size_t)u * K * kHeadDim + li * 8;
  float* sc_u = scores_ws + (size_t)v * K;
  float qb[8];
  {
    float4 a[kRowsInFlight][2];
#pragma unroll
    for (int t = 0; t < kRowsInFlight; ++t) {
      const int j = j_lo + grp + t * kSelGroups;
      if (j < j_hi) {
        a[t][0] = *reinterpret_cast<const float4*>(mu_u + (size_t)j * kHeadDim);
        a[t][1] = *reinterpret_cast<const float4*>(mu_u + (size_t)j * kHeadDim + 4);
      } else {
        a[t][0] = a[t][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    // the query sum while the centroid rows are in flight, made once per
    // workgroup by lanes 0-15 of wave 0 and handed over in LDS (every thread
    // loading every head's slice moved G x 16 KB through the load pipe)
    if (tid < 16) {
      float qs[8];
      qbar8(q, v, G, li, qs);
      *reinterpret_cast<float4*>(&qbar_lds[li * 8]) = make_float4(qs[0], qs[1], qs[2], qs[3]);
      *reinterpret_cast<float4*>(&qbar_lds[li * 8 + 4]) = make_float4(qs[4], qs[5], qs[6], qs[7]);
    }
    lds_barrier();
    {
      const float4 q0 = *reinterpret_cast<const float4*>(&qbar_lds[li * 8]);
      const float4 q1 = *reinterpret_cast<const float4*>(&qbar_lds[li * 8 + 4]);
      qb[0] = q0.x; qb[1] = q0.y; qb[2] = q0.z; qb[3] = q0.w;
      qb[4] = q1.x; qb[5] = q1.y; qb[6] = q1.z; qb[7] = q1.w;
    }
#pragma unroll
    for (int t = 0; t < kRowsInFlight; ++t) {
      const int j = j_lo + grp + t * kSelGroups;
      float d = qb[0] * a[t][0].x;
      d = fmaf(qb[1], a[t][0].y, d); d = fmaf(qb[2], a[t][0].z, d); d = fmaf(qb[3], a[t][0].w, d);
      d = fmaf(qb[4], a[t][1].x, d); d = fmaf(qb[5], a[t][1].y, d); d = fmaf(qb[6], a[t][1].z, d);
      d = fmaf(qb[7], a[t][1].w, d);
      d = sum16(d);
      if (li == 0 && j < j_hi) __hip_atomic_store(&sc_u[j], d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // this workgroup's stores are complete before the arrival count moves
  drain_memory_ops();
  lds_barrier();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&counters[v], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == (uint32_t)(nsplit - 1) ? 1 : 0;
  }
  lds_barrier();
  if (!sh_last) return;
  if (tid == 0) __hip_atomic_store(&counters[v], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ws.bw[tid] = 0;
  ws.bc[tid] = 0;
  {
    float mn = INFINITY, mx = -INFINITY;
    if (tid < K) {
      const float d = __hip_atomic_load(&sc_u[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int nsz = off[tid + 1] - off[tid];
      sz[tid] = nsz;
      csc[tid] = d;
      key[tid] = nsz > 0 ? score_key(d) : 0u;  // empty clusters rank below every score
      if (nsz > 0) mn = mx = d;
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      ws.rmin[wave] = mn;
      ws.rmax[wave] = mx;
    }
  }
  lds_barrier();

  // ---- phase 2: which clusters are taken whole, the cut, and the output
  // layout (exclusive scan of the taken amounts in index order)
  {
    int st[1] = {2};
    bool fast = true;
    if (m > budget) {
      float lo, scale;
      fast = score_range(ws, &lo, &scale) && block_select<kSelThreads, 1, false>(csc, key, sz, K, beff, lo, scale, ws, st);
    } else if (tid == 0) {
      ws.hdr[4] = -1;
      ws.hdr[5] = 0;
    }
    if (!fast) {
      // degenerate scores or a crowded crossing bucket: weighted radix select
      // on the keys by wave 0, then the walk among equal keys
      if (wave == 0) {
        uint32_t T = 0;
        int rem, cut = -1, need = 0;
        wave_radix_select<true>(key, sz, K, beff, hist, &T, &rem);
        int run = 0;
        for (int j0 = 0; j0 < K; j0 += kWave) {
          const int j = j0 + lane;
          const bool eq = j < K && key[j] == T;
          const int w = eq ? sz[j] : 0;
          const int incl = run + wave_incl_scan(w);
          const bool hit = eq && incl > rem && incl - w <= rem;
          const unsigned long long bb = __ballot(hit);
          if (bb) {
            const int src = (int)__ffsll((long long)bb) - 1;
            cut = __builtin_amdgcn_readlane(j, src);
            need = rem - __builtin_amdgcn_readlane(incl - w, src);
            break;
          }
          run = __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        for (int j = lane; j < K; j += kWave) {
          const uint32_t k = key[j];
          take[j] = sz[j] > 0 && (k > T || (k == T && j < cut)) ? 2 : (j == cut && need > 0 ? 1 : 0);
        }
        if (lane == 0) {
          ws.hdr[4] = need > 0 ? cut : -1;
          ws.hdr[5] = need;
        }
      }
      lds_barrier();
      st[0] = tid < K ? take[tid] : 0;
    }
    // the amounts: whole clusters, and the cut's share (known to its owner)
    const int j = tid;
    int amt = 0;
    if (j < K) amt = st[0] == 2 ? sz[j] : (st[0] == 1 ? ws.hdr[5] : 0);
    int total;
    const int incl = block_incl_scan<kSelThreads>(amt, ws.scr, &total);
    if (j < K) {
      ost[j] = incl - amt;
      take[j] = st[0] == 2 ? amt : 0;
    }
  }
  lds_barrier();
  const int cut = ws.hdr[4];
  const int need = ws.hdr[5];
  const bool fill = cut >= 0;
  const int n_cut = fill ? sz[cut] : 0;
  const int lo_cut = fill ? off[cut] : 0;

  // ---- phase 3 (waves 0-7): scores q_bar . k of the cut cluster's tokens (and
  // their range).  Meanwhile phase 5 (waves 8-15) writes the whole clusters, so
  // those stores overlap the wait for the cut cluster's rows.
  constexpr int kCutWaves = kSelWaves / 2;
  constexpr int kCutGroups = kCutWaves * (kWave / 16);
  constexpr int kCutRows = 8;
  const uint16_t* kc = k_clu + ((size_t)u * clu_stride + lo_cut) * kHeadDim + li * 8;
  uint32_t* cut_keys_g = cut_ws + (size_t)v * clu_stride;
  int32_t* out = sel_pos + (size_t)v * budget;
  if (wave < kCutWaves) {
    float mn = INFINITY, mx = -INFINITY;
    for (int r0 = 0; r0 < n_cut; r0 += kCutRows * kCutGroups) {
      uint4 cw[kCutRows];
#pragma unroll
      for (int t = 0; t < kCutRows; ++t) {
        const int i = r0 + grp + t * kCutGroups;
        cw[t] = i < n_cut ? *reinterpret_cast<const uint4*>(kc + (size_t)i * kHeadDim) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < kCutRows; ++t) {
        const int i = r0 + grp + t * kCutGroups;
        float d = qb[0] * bf16_lo(cw[t].x);
        d = fmaf(qb[1], bf16_hi(cw[t].x), d); d = fmaf(qb[2], bf16_lo(cw[t].y), d);
        d = fmaf(qb[3], bf16_hi(cw[t].y), d); d = fmaf(qb[4], bf16_lo(cw[t].z), d);
        d = fmaf(qb[5], bf16_hi(cw[t].z), d); d = fmaf(qb[6], bf16_lo(cw[t].w), d);
        d = fmaf(qb[7], bf16_hi(cw[t].w), d);
        d = sum16(d);
        if (li == 0 && i < n_cut) {
          mn = fminf(mn, d);
          mx = fmaxf(mx, d);
          if (n_cut <= kCutLds) {
            tkey[i] = score_key(d);
            tsc[i] = d;
          } else {
            cut_keys_g[i] = score_key(d);
          }
        }
      }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      ws.rmin[wave] = mn;
      ws.rmax[wave] = mx;
    }
  } else {
    if (lane == 0) {
      ws.rmin[wave] = INFINITY;
      ws.rmax[wave] = -INFINITY;
    }
    // ---- phase 5: whole clusters (positions off_j .. off_j + n_j - 1 at ost_j,
    // 64 consecutive slots per store instruction)
    for (int jb = (wave - kCutWaves) * kWave; jb < K; jb += (kSelWaves - kCutWaves) * kWave) {
      const int j = jb + lane;
      const int t = j < K ? take[j] : 0;
      const int o = j < K ? ost[j] : 0;
      const int lo2 = j < K ? off[j] : 0;
      unsigned long long live = __ballot(t > 0);
      while (live) {
        const int l = (int)__ffsll((long long)live) - 1;
        live &= live - 1;
        const int tl = __builtin_amdgcn_readlane(t, l), ol = __builtin_amdgcn_readlane(o, l);
        const int ll = __builtin_amdgcn_readlane(lo2, l);
        for (int i = lane; i < tl; i += kWave) out[ol + i] = ll + i;
      }
    }
  }
  if (n_cut > kCutLds) __threadfence_block();  // the wave-0 fallback below re-reads cut_keys_g
  lds_barrier();

  // ---- phase 4: the need highest-scoring tokens of the cut cluster, written
  // in position order (4 consecutive tokens per thread)
  if (fill) {
    constexpr int E = kCutLds / kSelThreads;
    int st[E];
    float lo, scale;
    const bool tok_fast = n_cut <= kCutLds && score_range(ws, &lo, &scale) &&
                          block_select<kSelThreads, E, true>(tsc, tkey, nullptr, n_cut, need, lo, scale, ws, st);
    if (tok_fast) {
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += st[e] == 2 ? 1 : 0;
      int total;
      int o = ost[cut] + block_incl_scan<kSelThreads>(cnt, ws.scr, &total) - cnt;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (st[e] == 2) out[o++] = lo_cut + tid * E + e;
    } else if (wave == 0) {
      if (n_cut <= kCutLds)
        fill_cut(tkey, n_cut, need, lo_cut, ost[cut], hist, out);
      else
        fill_cut(cut_keys_g, n_cut, need, lo_cut, ost[cut], hist, out);
    }
  }

  if (tid == 0) sel_count[v] = beff;
}

hipError_t launch_select(const uint16_t* q, int group, const float* cmean, const int32_t* offsets,
                         int K, const uint16_t* k_clu, int clu_stride, int budget, int32_t* sel_pos,
                         int32_t* sel_count, float* scores_ws, uint32_t* cut_ws, uint32_t* counters,
                         const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_tok, uint16_t* v_tok,
                         int capacity, int row, int units, int per_head, hipStream_t s) {
  // per_head: one recall per query head (group selections per unit, each from its own q_g)
  const int hs = per_head ? group : 1;
  const int sets = units * hs;
  const int need = (K + kSelRowsPerWg - 1) / kSelRowsPerWg;  // <= 4 for K <= 1024
  int nsplit = (256 + sets - 1) / sets;
  if (nsplit > kSelSplitMax) nsplit = kSelSplitMax;
  if (nsplit < need) nsplit = need;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)(sets * nsplit)), dim3(kSelThreads), 0, s, q,
                     per_head ? 1 : group, cmean, offsets, K, k_clu, clu_stride, budget, sel_pos, sel_count,
                     scores_ws, cut_ws, counters, k_new, v_new, k_tok, v_tok, capacity, row, hs, nsplit);
  return hipGetLastError();
}

}  // namespace ckv
