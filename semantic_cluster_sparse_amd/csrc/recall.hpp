// Building blocks of cluster-granularity recall (ClusterKV article,
// "大模型KV Cache压缩技术：ClusterKV的语义空间优化", §3.3), shared by the recall
// kernel and the fused recall + decode kernel: order-preserving score keys,
// wave-level weighted radix selects, the group query sum, and a block-level
// weighted selection over bucketed scores for a workgroup of NT threads.
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
// wave-synchronous weighted radix select on the keys.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace ckv {

constexpr int kCutLds = 4096;  // cut-cluster token keys kept in LDS up to this size

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

// The same sum in two parts: qrows_load issues the GT (>= G) row loads with
// no condition on G (rows past G - 1 repeat the last), so that a caller can
// issue more loads behind them and the sum waits for these alone; qbar_sum
// adds heads 0 .. G - 1 in order, the operations of qbar8.
template <int GT>
__device__ __forceinline__ void qrows_load(const uint16_t* q, int u, int G, int li, uint4 (&w)[GT]) {
#pragma unroll
  for (int h = 0; h < GT; ++h)
    w[h] = *reinterpret_cast<const uint4*>(q + ((size_t)u * G + min(h, G - 1)) * kHeadDim + li * 8);
}
template <int GT>
__device__ __forceinline__ void qbar_sum(const uint4 (&w)[GT], int G, float* qb) {
#pragma unroll
  for (int e = 0; e < 8; ++e) qb[e] = 0.f;
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const bool on = h < G;
    qb[0] = on ? qb[0] + bf16_lo(w[h].x) : qb[0]; qb[1] = on ? qb[1] + bf16_hi(w[h].x) : qb[1];
    qb[2] = on ? qb[2] + bf16_lo(w[h].y) : qb[2]; qb[3] = on ? qb[3] + bf16_hi(w[h].y) : qb[3];
    qb[4] = on ? qb[4] + bf16_lo(w[h].z) : qb[4]; qb[5] = on ? qb[5] + bf16_hi(w[h].z) : qb[5];
    qb[6] = on ? qb[6] + bf16_lo(w[h].w) : qb[6]; qb[7] = on ? qb[7] + bf16_hi(w[h].w) : qb[7];
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

// Inclusive prefix sum over the NT threads of the block; scr needs NT / 64
// ints.  The caller separates two uses of scr with a barrier.
template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int* scr, int* total) {
  constexpr int kWaves = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == kWave - 1) scr[wave] = x;
  lds_barrier();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = scr[w];
    pre += w < wave ? t : 0;
    tot += t;
  }
  *total = tot;
  return pre + x;
}

// Two inclusive prefix sums at once over the NT threads (one barrier); scr
// needs 2 * NT / 64 ints.  The caller separates two uses of scr with a barrier.
template <int NT>
__device__ __forceinline__ void block_incl_scan2(int a, int b, int* scr, int* ia, int* ib, int* ta, int* tb) {
  constexpr int kWaves = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int xa = wave_incl_scan(a);
  const int xb = wave_incl_scan(b);
  if (lane == kWave - 1) {
    scr[wave] = xa;
    scr[kWaves + wave] = xb;
  }
  lds_barrier();
  int pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int va = scr[w], vb = scr[kWaves + w];
    pa += w < wave ? va : 0;
    pb += w < wave ? vb : 0;
    sa += va;
    sb += vb;
  }
  *ia = pa + xa;
  *ib = pb + xb;
  *ta = sa;
  *tb = sb;
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

// LDS scratch of one block selection by NT threads.
template <int NT>
struct SelScratch {
  int bw[kBuckets];                 // bucket weights  } zero between selections
  int bc[kBuckets];                 // bucket counts   }
  float rmin[NT / kWave], rmax[NT / kWave];
  int scr[2 * NT / kWave];
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
template <int NT>
__device__ __forceinline__ bool score_range(const SelScratch<NT>& ws, float* lo, float* scale) {
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < NT / kWave; ++v) {
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
template <int NT, int E, bool UNIT>
__device__ __forceinline__ bool block_select(const float* sc, const uint32_t* key, const int* w, int n,
                                             int budget, float lo, float scale, SelScratch<NT>& ws, int (&st)[E]) {
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
  // descending scan: thread t holds buckets kBuckets-1-BPT t .. kBuckets-BPT (t+1)
  constexpr int BPT = kBuckets / NT;
  static_assert(BPT * NT == kBuckets, "buckets split evenly over the threads");
  int bv[BPT], bn[BPT], tsum = 0;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int bt = kBuckets - 1 - (BPT * tid + k);
    bv[k] = ws.bw[bt];
    bn[k] = ws.bc[bt];
    tsum += bv[k];
  }
  int total;
  int run = block_incl_scan<NT>(tsum, ws.scr, &total) - tsum;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int bt = kBuckets - 1 - (BPT * tid + k);
    const int before = run;
    run += bv[k];
    if (bv[k] > 0 && before <= budget && budget < run) {
      ws.hdr[0] = bt;
      ws.hdr[1] = before;
      ws.hdr[2] = bn[k];
      ws.hdr[3] = 0;
    }
    ws.bw[bt] = 0;  // re-arm for the next selection
    ws.bc[bt] = 0;
  }
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

}  // namespace ckv
