// Cluster-granularity recall (ClusterKV article, "大模型KV Cache压缩技术：
// ClusterKV的语义空间优化", §3.3; §3.1 motivates ranking clusters by q.mu).
//
// Per unit (one KV head of one sequence): q_bar = sum of the group's query
// heads; cluster score s_j = q_bar . mu_j (an empty cluster never scores);
// clusters in descending score (ties: smaller j) are taken whole while they
// fit; the first that does not fit contributes its highest q_bar.k tokens
// (ties: smaller position) so exactly min(budget, m) tokens are recalled.
//
// The walk in score order is a weighted selection: the clusters before the
// cut (in descending score) are taken whole, the cut cluster gives what is
// left of the budget.  It is found without sorting.  Scores are bucketed
// linearly between their min and max (1024 buckets, a monotone map); a block
// scan of the bucket weights in descending order finds the bucket where the
// running size crosses the budget; only the few clusters inside that bucket
// are ranked exactly (order-preserving 32-bit score keys, ties to the smaller
// index).  The partial fill inside the cut cluster is the same selection with
// unit weights over the q_bar.k scores of its tokens.  A crossing bucket with
// more than 64 members, or a degenerate score range, falls back to a
// wave-synchronous weighted radix select on the keys.  Several workgroups of
// 1024 threads per recalled set (4 up to 64 sets, then about 256 per launch,
// never fewer than K / 256) each score a share of the clusters; the last of
// them to finish (device-scope arrival counter) makes the selection.
// A set is one KV head's recall (q_bar over its G query heads) or, in the
// per-query-head mode, one query head's (q_g alone).  The barriers wait on LDS
// only, so global loads stay in flight across them.  Recalled positions are
// written by whole waves, 64 consecutive slots per store instruction.
#include "common.hpp"
#include "launch.hpp"

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
  // every head's load in flight at once, then the sum in head order
  uint4 w[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h)
    w[h] = h < G ? *reinterpret_cast<const uint4*>(q + ((size_t)u * G + h) * kHeadDim + li * 8)
                 : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 8; ++e) qb[e] = 0.f;
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      qb[0] += bf16_lo(w[h].x); qb[1] += bf16_hi(w[h].x);
      qb[2] += bf16_lo(w[h].y); qb[3] += bf16_hi(w[h].y);
      qb[4] += bf16_lo(w[h].z); qb[5] += bf16_hi(w[h].z);
      qb[6] += bf16_lo(w[h].w); qb[7] += bf16_hi(w[h].w);
    }
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

// ---------------------------------------------------------------------------
// Block-level pieces (1024 threads).
// ---------------------------------------------------------------------------
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBuckets = 1024;
constexpr int kMaxCand = 64;

// Barrier that waits for this thread's LDS operations only: global loads stay
// in flight across it.  The memory clobbers keep the compiler from moving
// memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();  // convergent: never duplicated into divergent code
  asm volatile("" ::: "memory");
}

// Inclusive prefix sum over the 1024 threads; scr needs kSelWaves ints.  The
// caller separates two uses of scr with a barrier.
__device__ __forceinline__ int block_incl_scan(int v, int* scr, int* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == kWave - 1) scr[wave] = x;
  lds_barrier();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = scr[w];
    pre += w < wave ? t : 0;
    tot += t;
  }
  *total = tot;
  return pre + x;
}

// Min / max over the 64 lanes of a wave (DPP within rows of 16, then the four
// row results through readlane); the result is wave-uniform.
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp_f32<kDppXor1>(v));
  v = fminf(v, dpp_f32<kDppXor2>(v));
  v = fminf(v, dpp_f32<kDppHalfMirror>(v));
  v = fminf(v, dpp_f32<kDppMirror>(v));
  const int x = __float_as_int(v);
  return fminf(fminf(__int_as_float(__builtin_amdgcn_readlane(x, 0)), __int_as_float(__builtin_amdgcn_readlane(x, 16))),
               fminf(__int_as_float(__builtin_amdgcn_readlane(x, 32)), __int_as_float(__builtin_amdgcn_readlane(x, 48))));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  const int x = __float_as_int(v);
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(x, 0)), __int_as_float(__builtin_amdgcn_readlane(x, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(x, 32)), __int_as_float(__builtin_amdgcn_readlane(x, 48))));
}

// LDS scratch of one block selection.
struct SelScratch {
  int bw[kBuckets];                 // bucket weights  } zero between selections
  int bc[kBuckets];                 // bucket counts   }
  float rmin[kSelWaves], rmax[kSelWaves];
  int scr[kSelWaves];
  int cand[kMaxCand];
  int rs_w[kMaxCand], rs_i[kMaxCand];
  int hdr[8];                       // crossing bucket, weight above it, its count, candidates, cut, need
  unsigned char dec[kCutLds];       // state of the crossing bucket's members (several-member case)
};

// Monotone map of a score in [lo, lo + range] to a bucket in [0, kBuckets).
__device__ __forceinline__ int score_bucket(float v, float lo, float scale) {
  const float x = (v - lo) * scale;
  return x < (float)(kBuckets - 1) ? (int)x : kBuckets - 1;
}

// Score range from the per-wave partials in ws.rmin / ws.rmax; false if it is
// degenerate (all equal, or not finite).
__device__ __forceinline__ bool score_range(const SelScratch& ws, float* lo, float* scale) {
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < kSelWaves; ++v) {
    mn = fminf(mn, ws.rmin[v]);
    mx = fmaxf(mx, ws.rmax[v]);
  }
  const float range = mx - mn;
  const float sc = (float)kBuckets / range;
  *lo = mn;
  *scale = sc;
  return range > 0.f && range < INFINITY && sc > 0.f && sc < INFINITY;
}

// Descending weighted selection by the whole block over n <= E * 1024
// elements held in LDS: scores sc[i] (finite), order-preserving keys key[i],
// weights w[i] (unit if UNIT; weight 0 never counts); thread t owns elements
// E t .. E t + E - 1.  Walking the elements by (key desc, index asc) with
// running weight R before element e, the state of e is 2 if R + w_e <=
// budget, 1 if R < budget < R + w_e (it gets budget - R), 0 otherwise.
// Requires total counted weight > budget >= 0, a non-degenerate score range
// (lo, scale from score_range) and ws.bw / ws.bc zero; leaves them zero.
// The scores are bucketed linearly; a block scan over the buckets in
// descending order finds the bucket where the running weight crosses the
// budget.  When that bucket has a single member (the usual case) its state
// follows at once; otherwise its members (at most kMaxCand) are ranked
// exactly by wave 0.  st[e] receives the states of this thread's elements; the
// state-1 element and its share land in ws.hdr[4], ws.hdr[5] (-1 / 0 if
// none), readable after the caller's next barrier.  Returns false
// (block-uniform) when the crossing bucket has more than kMaxCand members.
template <int E, bool UNIT>
__device__ __forceinline__ bool block_select(const float* sc, const uint32_t* key, const int* w, int n,
                                             int budget, float lo, float scale, SelScratch& ws, int (&st)[E]) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  int b[E], wt[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid * E + e;
    const int wi = i < n ? (UNIT ? 1 : w[i]) : 0;
    wt[e] = wi > 0 ? wi : 0;
    b[e] = wt[e] > 0 ? score_bucket(sc[i], lo, scale) : -1;
    if (wt[e] > 0) {
      atomicAdd(&ws.bw[b[e]], wt[e]);
      atomicAdd(&ws.bc[b[e]], 1);
    }
  }
  if (tid == 0) {
    ws.hdr[4] = -1;
    ws.hdr[5] = 0;
  }
  lds_barrier();
  // descending scan: thread t holds bucket kBuckets-1-t
  const int bt = kBuckets - 1 - tid;
  const int v = ws.bw[bt];
  const int cb = ws.bc[bt];
  int total;
  const int incl = block_incl_scan(v, ws.scr, &total);
  if (v > 0 && incl - v <= budget && budget < incl) {
    ws.hdr[0] = bt;
    ws.hdr[1] = incl - v;
    ws.hdr[2] = cb;
    ws.hdr[3] = 0;
  }
  ws.bw[bt] = 0;  // re-arm for the next selection
  ws.bc[bt] = 0;
  lds_barrier();
  const int bstar = ws.hdr[0], above = ws.hdr[1], nb = ws.hdr[2];
  if (nb == 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (b[e] != bstar) {
        st[e] = b[e] > bstar ? 2 : 0;
      } else {
        st[e] = above + wt[e] <= budget ? 2 : (above < budget ? 1 : 0);
        if (st[e] == 1) {
          ws.hdr[4] = tid * E + e;
          ws.hdr[5] = budget - above;
        }
      }
    }
    return true;
  }
  if (nb > kMaxCand) return false;
  // several members: exact order inside the crossing bucket, rank by (key desc, index asc)
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (b[e] == bstar) ws.cand[atomicAdd(&ws.hdr[3], 1)] = tid * E + e;
  lds_barrier();
  if (wave == 0) {
    const int ci = lane < nb ? ws.cand[lane] : 0;
    const uint32_t ck = lane < nb ? key[ci] : 0u;
    int rank = 0;
    for (int l = 0; l < nb; ++l) {
      const uint32_t kl = (uint32_t)__builtin_amdgcn_readlane((int)ck, l);
      const int il = __builtin_amdgcn_readlane(ci, l);
      rank += (kl > ck || (kl == ck && il < ci)) ? 1 : 0;
    }
    if (lane < nb) {
      ws.rs_w[rank] = UNIT ? 1 : w[ci];
      ws.rs_i[rank] = ci;
    }
    const int wr = lane < nb ? ws.rs_w[lane] : 0;
    const int ir = lane < nb ? ws.rs_i[lane] : 0;
    const int rrun = above + wave_incl_scan(wr) - wr;  // weight before this rank
    if (lane < nb) {
      const int s2 = rrun + wr <= budget ? 2 : (rrun < budget ? 1 : 0);
      ws.dec[ir] = (unsigned char)s2;
      if (s2 == 1) {
        ws.hdr[4] = ir;
        ws.hdr[5] = budget - rrun;
      }
    }
  }
  lds_barrier();
#pragma unroll
  for (int e = 0; e < E; ++e) st[e] = b[e] != bstar ? (b[e] > bstar ? 2 : 0) : (int)ws.dec[tid * E + e];
  return true;
}

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
  __shared__ __attribute__((aligned(16))) SelScratch ws;
  __shared__ int sh_cut, sh_need, sh_last;

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
    // the query sum while the centroid rows are in flight
    qbar8(q, v, G, li, qb);
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
      fast = score_range(ws, &lo, &scale) && block_select<1, false>(csc, key, sz, K, beff, lo, scale, ws, st);
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
    const int incl = block_incl_scan(amt, ws.scr, &total);
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
                          block_select<E, true>(tsc, tkey, nullptr, n_cut, need, lo, scale, ws, st);
    if (tok_fast) {
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += st[e] == 2 ? 1 : 0;
      int total;
      int o = ost[cut] + block_incl_scan(cnt, ws.scr, &total) - cnt;
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
