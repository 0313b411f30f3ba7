// Fused recall + sparse decode: one launch per layer and decode step that
// recalls the clusters of every attended set and attends to the recalled rows
// (ClusterKV article, "大模型KV Cache压缩技术：ClusterKV的语义空间优化", §3.3
// selection procedure, §3.1 attention over the recalled tokens, §4.1
// cluster-contiguous rows; ClusterKV abstract, arXiv 2412.03213: recall at
// semantic-cluster granularity).
//
// Each attended set (one KV head with its group-summed query, or one query
// head) is split into W chunks of its attended rows, one workgroup each.
// Every workgroup of a set recalls the whole set itself: it scores all K
// centroids (q_bar . mu_j), makes the same weighted selection (recall.hpp) and
// so knows, without any exchange with the others, which clusters are taken
// whole, which cluster is cut and how many of its tokens are kept.  The
// attended rows are laid out as one list per set,
//   sinks | recent rows | whole clusters in index order | the cut's tokens,
// whose length n_sink + r + min(budget, m) does not depend on the recall, so
// each workgroup knows its chunk from the start.  Only a workgroup whose chunk
// reaches the cut's tokens scores them (q_bar . k) and picks the best ones.
// Whole-cluster rows are runs of the cluster-ordered copy located by a search
// over the taken clusters' running row counts.  The recalled positions are
// also written out (sel_pos, ascending, as ckv_select writes them), each by
// the workgroup that streams that row.  Streaming and the split-K merge are
// the decode's (stream.hpp).
//
// The W workgroups of a set are placed on one XCD (workgroups are dispatched
// to the 8 XCDs in turn), so the set's centroids, which each of them reads,
// come from that XCD's L2 after the first miss.  The chunk owning the cut
// cluster gets fewer rows, since it scores the cut cluster first.  With a
// prefetch hint (the next layer's centroids and offsets, same shape), the
// chunks that do not merge read the next call's centroids of their unit into
// the XCD's L2 while the last one merges.
#include "recall.hpp"
#include "stream.hpp"

namespace ckv {

constexpr int kRdThreads = kDecThreads;        // 512: the streaming shape
constexpr int kRdWaves = kRdThreads / kWave;
constexpr int kRdGroups = kRdThreads / 16;     // 16-lane centroid-row groups
constexpr int kRdRowsInFlight = 16;            // centroid rows per group per load round
constexpr int kRdClu = kMaxClusters / kRdThreads;  // clusters per thread in the selection
constexpr int kRdTok = kCutLds / kRdThreads;       // cut tokens per thread in the selection
constexpr int kAfterCut = 0x40000000;          // whole cluster with an index above the cut's
// Rows an even share of the chunk owning the cut gives up: its workgroup first
// loads and scores the cut cluster's keys and selects among them, which takes
// about as long as streaming this many rows.
constexpr int kCutPenaltyRows = 320;
static_assert(kRdClu * kRdThreads == kMaxClusters && kRdTok * kRdThreads == kCutLds, "even split");

// LDS of the recall phase; it lives in the decode ring, which is free until
// the first row is streamed.
struct RecallScratch {
  float csc[kMaxClusters];
  uint32_t key[kMaxClusters];
  int sz[kMaxClusters];
  int take[kMaxClusters];
  int hist[kHistCopies * kHistBins];
  uint32_t tkey[kCutLds];
  float tsc[kCutLds];
  SelScratch<kRdThreads> ws;
};
static_assert(sizeof(RecallScratch) <= kRingBytes, "recall scratch fits in the ring");

template <int GT>
__global__ __launch_bounds__(kRdThreads) void recall_decode_kernel(
    const uint16_t* __restrict__ q, int G, const float* __restrict__ cmean, const int32_t* __restrict__ offsets,
    int K, uint16_t* k_tok, uint16_t* v_tok, int capacity, const uint16_t* __restrict__ k_clu,
    const uint16_t* __restrict__ v_clu, int clu_stride, int budget, int n_sink, int n_clustered, int n_total,
    int32_t* __restrict__ sel_pos, int32_t* __restrict__ sel_count, float* __restrict__ partials,
    uint32_t* __restrict__ counters, uint32_t* __restrict__ cut_ws, float* __restrict__ out,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, const float* __restrict__ pf_cmean,
    const int32_t* __restrict__ pf_offsets, int hs, int W) {
  // ring (recall scratch before the stream, merge area after it) | row sources
  __shared__ __attribute__((aligned(16))) unsigned char smem[kRingBytes + kRowSegment * 4];
  static_assert(kDecWaves * GT * kPartialStride * 4 <= kRingBytes + kRowSegment * 4,
                "merge area must fit in the ring and row sources");
  __shared__ int wl_end[kMaxClusters];  // running row count through the t-th whole cluster
  __shared__ int wl_off[kMaxClusters];  // its first position, | kAfterCut above the cut
  __shared__ int sh[8];
  __shared__ __attribute__((aligned(16))) float qbar_lds[kHeadDim];  // the group's query sum
  RecallScratch& rs = *reinterpret_cast<RecallScratch*>(smem);
  SelScratch<kRdThreads>& ws = rs.ws;
  int* rowsrc = reinterpret_cast<int*>(smem + kRingBytes);

  // workgroup -> (set, chunk), the W chunks of a set on one XCD
  const int nwg = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  const int xcd = b & 7, per = nwg >> 3, extra = nwg & 7;
  const int lg = xcd * per + min(xcd, extra) + (b >> 3);
  const int v = lg / W;       // attended set
  const int w = lg - v * W;   // chunk
  const int u = v / hs;       // unit (hs = 1: set = unit; hs = G: one set per query head)

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int li = tid & 15;
  const int grp = tid >> 4;

  // the stream's query operand, loaded while the recall's loads are in flight
  StreamState sst;
  stream_init(sst, q, v, G);
  // ---- recall, step 1: every cluster's score q_bar . mu_j (16 lanes per
  // centroid row, up to 512 rows in flight per round) and size
  const int32_t* off = offsets + (size_t)u * (K + 1);
  int offr[kRdClu + 1];
#pragma unroll
  for (int e = 0; e <= kRdClu; ++e) offr[e] = off[min(kRdClu * tid + e, K)];
  const int m = off[K];
  const int beff = budget < m ? budget : m;
  const float* mu_u = cmean + (size_t)u * K * kHeadDim + li * 8;
  // The query sum is made once per workgroup, by lanes 0-15 of wave 0 (one
  // 16-byte slice of every head each), and handed to the other threads in
  // LDS.  (Every thread loading every head's slice moved G x 16 KB per
  // workgroup through its load pipe for a 4 KB query and, at G = 16, held the
  // centroid rows back by ~1.2 us.)  The makers issue their query loads before
  // their centroid rows' and sum behind them: a wave's loads complete in order.
  const bool qmaker = tid < 16;
  uint4 qw[GT];
  if (qmaker) qrows_load<GT>(q, v, G, li, qw);
  constexpr int kRound = kRdGroups * kRdRowsInFlight;
  float4 a[kRdRowsInFlight][2];
#pragma unroll
  for (int t = 0; t < kRdRowsInFlight; ++t) {  // rows past K - 1 repeat the last; their scores are dropped
    const int j = min(grp + t * kRdGroups, K - 1);
    a[t][0] = *reinterpret_cast<const float4*>(mu_u + (size_t)j * kHeadDim);
    a[t][1] = *reinterpret_cast<const float4*>(mu_u + (size_t)j * kHeadDim + 4);
  }
  __builtin_amdgcn_sched_barrier(0);  // the sum (and its wait) stays behind the row loads
  if (qmaker) {
    float qs[8];
    qbar_sum<GT>(qw, G, qs);
    *reinterpret_cast<float4*>(&qbar_lds[li * 8]) = make_float4(qs[0], qs[1], qs[2], qs[3]);
    *reinterpret_cast<float4*>(&qbar_lds[li * 8 + 4]) = make_float4(qs[4], qs[5], qs[6], qs[7]);
  }
  lds_barrier();
  float qb[8];
  {
    const float4 q0 = *reinterpret_cast<const float4*>(&qbar_lds[li * 8]);
    const float4 q1 = *reinterpret_cast<const float4*>(&qbar_lds[li * 8 + 4]);
    qb[0] = q0.x; qb[1] = q0.y; qb[2] = q0.z; qb[3] = q0.w;
    qb[4] = q1.x; qb[5] = q1.y; qb[6] = q1.z; qb[7] = q1.w;
  }
  for (int j0 = 0;;) {
#pragma unroll
    for (int t = 0; t < kRdRowsInFlight; ++t) {
      const int j = j0 + grp + t * kRdGroups;
      float d = qb[0] * a[t][0].x;
      d = fmaf(qb[1], a[t][0].y, d); d = fmaf(qb[2], a[t][0].z, d); d = fmaf(qb[3], a[t][0].w, d);
      d = fmaf(qb[4], a[t][1].x, d); d = fmaf(qb[5], a[t][1].y, d); d = fmaf(qb[6], a[t][1].z, d);
      d = fmaf(qb[7], a[t][1].w, d);
      d = sum16(d);
      if (li == 0 && j < K) rs.csc[j] = d;
    }
    j0 += kRound;
    if (j0 >= K) break;
#pragma unroll
    for (int t = 0; t < kRdRowsInFlight; ++t) {
      const int j = min(j0 + grp + t * kRdGroups, K - 1);
      a[t][0] = *reinterpret_cast<const float4*>(mu_u + (size_t)j * kHeadDim);
      a[t][1] = *reinterpret_cast<const float4*>(mu_u + (size_t)j * kHeadDim + 4);
    }
  }
#pragma unroll
  for (int e = 0; e < kRdClu; ++e) {
    ws.bw[kRdClu * tid + e] = 0;
    ws.bc[kRdClu * tid + e] = 0;
  }
  lds_barrier();
  int szr[kRdClu];
  {
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < kRdClu; ++e) {
      const int j = kRdClu * tid + e;
      szr[e] = j < K ? offr[e + 1] - offr[e] : 0;
      if (j < K) {
        const float d = rs.csc[j];
        rs.sz[j] = szr[e];
        rs.key[j] = szr[e] > 0 ? score_key(d) : 0u;  // empty clusters rank below every score
        if (szr[e] > 0) {
          mn = fminf(mn, d);
          mx = fmaxf(mx, d);
        }
      }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      ws.rmin[wave] = mn;
      ws.rmax[wave] = mx;
    }
  }
  lds_barrier();

  // ---- recall, step 2: which clusters are taken whole, the cut and its share
  int st[kRdClu];
#pragma unroll
  for (int e = 0; e < kRdClu; ++e) st[e] = 2;
  {
    bool fast = true;
    if (m > budget) {
      float lo, scale;
      fast = score_range(ws, &lo, &scale) &&
             block_select<kRdThreads, kRdClu, false>(rs.csc, rs.key, rs.sz, K, beff, lo, scale, ws, st);
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
        wave_radix_select<true>(rs.key, rs.sz, K, beff, rs.hist, &T, &rem);
        int run = 0;
        for (int j0 = 0; j0 < K; j0 += kWave) {
          const int j = j0 + lane;
          const bool eq = j < K && rs.key[j] == T;
          const int wj = eq ? rs.sz[j] : 0;
          const int incl = run + wave_incl_scan(wj);
          const bool hit = eq && incl > rem && incl - wj <= rem;
          const unsigned long long bb = __ballot(hit);
          if (bb) {
            const int src = (int)__ffsll((long long)bb) - 1;
            cut = __builtin_amdgcn_readlane(j, src);
            need = rem - __builtin_amdgcn_readlane(incl - wj, src);
            break;
          }
          run = __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        for (int j = lane; j < K; j += kWave) {
          const uint32_t k = rs.key[j];
          rs.take[j] = rs.sz[j] > 0 && (k > T || (k == T && j < cut)) ? 2 : (j == cut && need > 0 ? 1 : 0);
        }
        if (lane == 0) {
          ws.hdr[4] = need > 0 ? cut : -1;
          ws.hdr[5] = need;
        }
      }
      lds_barrier();
#pragma unroll
      for (int e = 0; e < kRdClu; ++e) st[e] = kRdClu * tid + e < K ? rs.take[kRdClu * tid + e] : 0;
    }
  }
  lds_barrier();
  const int cut = ws.hdr[4];
  const int need = ws.hdr[5];

  // whole clusters in index order: their compact list with running row counts
  int nw, T_whole;
  {
    int cw = 0, rw = 0;
    bool whole[kRdClu];
#pragma unroll
    for (int e = 0; e < kRdClu; ++e) {
      whole[e] = kRdClu * tid + e < K && st[e] == 2 && szr[e] > 0;
      cw += whole[e] ? 1 : 0;
      rw += whole[e] ? szr[e] : 0;
    }
    int ci, ri;
    block_incl_scan2<kRdThreads>(cw, rw, ws.scr, &ci, &ri, &nw, &T_whole);
    ci -= cw;
    ri -= rw;
#pragma unroll
    for (int e = 0; e < kRdClu; ++e) {
      const int j = kRdClu * tid + e;
      if (j == cut) {
        sh[0] = ri;       // whole rows before the cut cluster: its first recalled slot
        sh[1] = offr[e];  // its first position
        sh[2] = szr[e];   // its size
      }
      if (whole[e]) {
        ri += szr[e];
        wl_end[ci] = ri;
        wl_off[ci] = offr[e] | (cut >= 0 && j > cut ? kAfterCut : 0);
        ++ci;
      }
    }
  }
  if (w == 0 && tid == 0) sel_count[v] = beff;

  // this workgroup's chunk of the set's attended rows.  The last chunk holds
  // the cut cluster's kept tokens, and its workgroup first scores the whole
  // cut cluster, so it takes kCutPenaltyRows fewer rows than an even share.
  const int r_recent = n_total - n_clustered;
  const int R = n_sink + r_recent + beff;
  int c0 = 0, c1 = R;
  if (W > 1) {
    const int even = (R + W - 1) / W;
    const int tail = need > 0 ? max(need, even - kCutPenaltyRows) : even;
    // rounded down: the first W - 1 chunks end at or before R - tail, so
    // every cut row falls in the last chunk and no other workgroup scores
    // the cut cluster
    const int chunk = (R - tail) / (W - 1);
    c0 = min(w * chunk, R);
    c1 = w == W - 1 ? R : min(c0 + chunk, R);
  }
  const int wbase = n_sink + r_recent;  // first whole-cluster row of the list
  const int cbase = wbase + T_whole;    // first cut row
  int32_t* sp = sel_pos + (size_t)v * budget;
  lds_barrier();
  const int ost_cut = cut >= 0 ? sh[0] : 0;
  const int lo_cut = cut >= 0 ? sh[1] : 0;
  const int n_cut = cut >= 0 ? sh[2] : 0;

  // ---- recall, step 3 (only where the chunk reaches the cut's rows): the
  // cut cluster's token scores q_bar . k and the need best of them.  tok_st
  // holds the states of this thread's kRdTok consecutive tokens, tok_rank the
  // rank among the kept ones of its first kept token.
  int tok_st[kRdTok];
  int tok_rank = 0;
  bool cut_in_ws = false;  // the kept positions went to sel_pos instead (fallback)
#pragma unroll
  for (int e = 0; e < kRdTok; ++e) tok_st[e] = 0;
  if (need > 0 && c1 > cbase) {
    constexpr int kCutRows = 8;
    const uint16_t* kc = k_clu + ((size_t)u * clu_stride + lo_cut) * kHeadDim + li * 8;
    uint32_t* cut_keys_g = cut_ws + (size_t)v * clu_stride;
    float mn = INFINITY, mx = -INFINITY;
    for (int r0 = 0; r0 < n_cut; r0 += kCutRows * kRdGroups) {
      uint4 cw[kCutRows];
#pragma unroll
      for (int t = 0; t < kCutRows; ++t) {
        const int i = r0 + grp + t * kRdGroups;
        cw[t] = i < n_cut ? *reinterpret_cast<const uint4*>(kc + (size_t)i * kHeadDim) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < kCutRows; ++t) {
        const int i = r0 + grp + t * kRdGroups;
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
            rs.tkey[i] = score_key(d);
            rs.tsc[i] = d;
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
    if (n_cut > kCutLds) __threadfence_block();  // wave 0 re-reads cut_keys_g below
    lds_barrier();
    float lo, scale;
    const bool tok_fast = n_cut <= kCutLds && score_range(ws, &lo, &scale) &&
                          block_select<kRdThreads, kRdTok, true>(rs.tsc, rs.tkey, nullptr, n_cut, need, lo, scale,
                                                                 ws, tok_st);
    if (tok_fast) {
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < kRdTok; ++e) cnt += tok_st[e] == 2 ? 1 : 0;
      int total;
      lds_barrier();  // scr was last read inside the selection
      tok_rank = block_incl_scan<kRdThreads>(cnt, ws.scr, &total) - cnt;
    } else {
      // fallback: wave 0 writes the kept positions, in order, to sel_pos;
      // the row sources below read them back
      cut_in_ws = true;
#pragma unroll
      for (int e = 0; e < kRdTok; ++e) tok_st[e] = 0;
      if (wave == 0) {
        if (n_cut <= kCutLds)
          fill_cut(rs.tkey, n_cut, need, lo_cut, ost_cut, rs.hist, sp);
        else
          fill_cut(cut_keys_g, n_cut, need, lo_cut, ost_cut, rs.hist, sp);
      }
      __threadfence();
    }
  }
  __syncthreads();  // the recall scratch is dead: the ring is free

  // ---- decode: the chunk's rows, 1024 row sources at a time
  RowBases rb;
  rb.ktu = k_tok + (size_t)u * capacity * kHeadDim;
  rb.vtu = v_tok + (size_t)u * capacity * kHeadDim;
  rb.kcu = k_clu + (size_t)u * clu_stride * kHeadDim;
  rb.vcu = v_clu + (size_t)u * clu_stride * kHeadDim;
  rb.knu = k_new != nullptr ? k_new + (size_t)u * kHeadDim : rb.ktu;
  rb.vnu = v_new != nullptr ? v_new + (size_t)u * kHeadDim : rb.vtu;
  const int new_row = k_new != nullptr ? n_total - 1 : -1;
  constexpr int kSegPerThread = kRowSegment / kRdThreads;
  for (int seg = c0; seg < c1; seg += kRowSegment) {
    const int seg_end = min(c1, seg + kRowSegment);
    const int nrows = seg_end - seg;
    // the previous segment's rows are all streamed (the first segment follows
    // the barrier that ends the recall)
    if (seg != c0) __syncthreads();
    // sinks, recent rows and (fallback) the cut's rows: one thread per row
#pragma unroll
    for (int k = 0; k < kSegPerThread; ++k) {
      const int i = tid + k * kRdThreads;
      const int r = seg + i;
      if (i < nrows) {
        if (r < n_sink) {
          rowsrc[i] = r;
        } else if (r < wbase) {
          const int row = n_clustered + (r - n_sink);
          rowsrc[i] = row == new_row ? kNewFlag : row;
        } else if (r >= cbase && cut_in_ws) {
          const int p = __hip_atomic_load(&sp[ost_cut + (r - cbase)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          rowsrc[i] = min(max(p, 0), m - 1) | kCluFlag;
        }
      }
    }
    // whole clusters: runs of the cluster-ordered copy, one cluster per wave at a time
    const int a = max(seg, wbase) - wbase, bnd = min(seg_end, cbase) - wbase;
    if (a < bnd) {
      // first whole cluster whose rows reach past a (wl_end increases): lane l
      // looks at block l of 16 clusters, then at the clusters of the first block
      const int bi = min(16 * lane + 15, nw - 1);
      const unsigned long long b1 = __ballot(16 * lane < nw && wl_end[bi] > a);
      const int blk = b1 ? (int)__ffsll((long long)b1) - 1 : 0;
      const int ti = 16 * blk + (lane & 15);
      const unsigned long long b2 = __ballot(lane < 16 && ti < nw && wl_end[ti] > a);
      const int t0 = 16 * blk + (b2 ? (int)__ffsll((long long)b2) - 1 : 0);
      for (int t = t0 + wave; t < nw; t += kRdWaves) {
        const int start = t > 0 ? wl_end[t - 1] : 0;
        if (start >= bnd) break;
        const int end = wl_end[t];
        const int wo = wl_off[t];
        const int p0 = wo & ~kAfterCut;
        const int slot0 = (wo & kAfterCut) ? need : 0;
        const int lo = max(start, a), hi = min(end, bnd);
        for (int i = lo + lane; i < hi; i += kWave) {
          const int p = p0 + (i - start);
          rowsrc[i + wbase - seg] = p | kCluFlag;
          sp[i + slot0] = p;
        }
      }
    }
    // the cut's kept tokens, held as states by the threads that own them
    if (!cut_in_ws && need > 0 && seg_end > cbase) {
      int rk = tok_rank;
#pragma unroll
      for (int e = 0; e < kRdTok; ++e) {
        if (tok_st[e] == 2) {
          const int r = cbase + rk;
          if (r >= seg && r < seg_end) {
            const int p = lo_cut + kRdTok * tid + e;
            rowsrc[r - seg] = p | kCluFlag;
            sp[ost_cut + rk] = p;
          }
          ++rk;
        }
      }
    }
    __syncthreads();
    stream_rows(sst, rb, lds_addr(rowsrc), lds_addr(smem), nrows, G);
  }
  const int rank = finish_chunk<GT>(sst, reinterpret_cast<float*>(smem), &sh[7], partials, counters, out, v, w, W, G);

  // The appended token's row into the token-order cache (this launch streamed
  // it from k_new / v_new).  Done last: the copy's load would otherwise hold
  // up the wave's first recall loads.
  if (k_new != nullptr && w == 0 && v % hs == 0 && tid < 32) {
    const int c8 = (tid & 15) * 8;
    const uint16_t* src = (tid < 16 ? k_new : v_new) + (size_t)u * kHeadDim + c8;
    uint16_t* dst = (tid < 16 ? k_tok : v_tok) + ((size_t)u * capacity + n_total - 1) * kHeadDim + c8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }

  // The chunks that did not merge are done while the last one merges: they
  // bring the next call's centroids and offsets of this unit (the next layer,
  // laid out like this one) into this XCD's L2, which the next launch places
  // on the same XCD, so that its first phase reads them from there.
  if (pf_cmean != nullptr && rank < W - 1 && v % hs == 0) {
    const float4* src = reinterpret_cast<const float4*>(pf_cmean + (size_t)u * K * kHeadDim);
    const int n4 = K * (kHeadDim / 4);
    const int lo = (int)((long long)n4 * rank / (W - 1)), hi = (int)((long long)n4 * (rank + 1) / (W - 1));
    uint32_t acc = 0;
    for (int i0 = lo; i0 < hi; i0 += 8 * kRdThreads) {
      float4 f[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + tid + k * kRdThreads;
        f[k] = i < hi ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= __float_as_uint(f[k].x);
    }
    if (rank == 0) {
      const int32_t* po = pf_offsets + (size_t)u * (K + 1);
      for (int i = tid; i <= K; i += kRdThreads) acc ^= (uint32_t)po[i];
    }
    asm volatile("" ::"v"(acc));  // the loads must complete; their values are not needed
  }
}

int recall_decode_chunks(int sets, int rows) {
  // about 256 workgroups per launch (one per CU), chunks of at least 64 rows
  int W = (256 + sets - 1) / sets;
  if (W > kMaxChunks) W = kMaxChunks;
  const int wmax = (rows + 63) / 64;
  if (W > wmax) W = wmax;
  if (W < 1) W = 1;
  return W;
}

hipError_t launch_recall_decode(const uint16_t* q, int group, const float* cmean, const int32_t* offsets, int K,
                                uint16_t* k_tok, uint16_t* v_tok, int capacity, const uint16_t* k_clu,
                                const uint16_t* v_clu, int clu_stride, int budget, int n_sink, int n_clustered,
                                int n_total, int32_t* sel_pos, int32_t* sel_count, float* partials,
                                uint32_t* counters, uint32_t* cut_ws, float* out, const uint16_t* k_new,
                                const uint16_t* v_new, const float* pf_cmean, const int32_t* pf_offsets, int units,
                                int per_head, hipStream_t s) {
  const int hs = per_head ? group : 1;
  const int Ge = per_head ? 1 : group;
  const int sets = units * hs;
  const int m = n_clustered - n_sink;
  const int beff = budget < m ? budget : m;
  const int W = recall_decode_chunks(sets, n_sink + beff + (n_total - n_clustered));
  const dim3 grid((unsigned)(sets * W));
  int gt = 1;
  while (gt < Ge) gt <<= 1;
#define CKV_RD(GTV)                                                                                           \
  hipLaunchKernelGGL(recall_decode_kernel<GTV>, grid, dim3(kRdThreads), 0, s, q, Ge, cmean, offsets, K, k_tok, \
                     v_tok, capacity, k_clu, v_clu, clu_stride, budget, n_sink, n_clustered, n_total, sel_pos,  \
                     sel_count, partials, counters, cut_ws, out, k_new, v_new, pf_cmean, pf_offsets, hs, W)
  switch (gt) {
    case 1: CKV_RD(1); break;
    case 2: CKV_RD(2); break;
    case 4: CKV_RD(4); break;
    case 8: CKV_RD(8); break;
    default: CKV_RD(16); break;
  }
#undef CKV_RD
  return hipGetLastError();
}

}  // namespace ckv
