// Sparse decode: attention of every query head of a GQA group over the
// recalled rows only -- softmax(q K_S^T / sqrt(d)) V_S with S = sinks, the
// recalled clustered rows (cluster-ordered copy) and the recent unclustered
// rows (ClusterKV article, "大模型KV Cache压缩技术：ClusterKV的语义空间优化",
// §3.1 attention formula; §4.1 cluster-contiguous storage; ClusterKV
// abstract, arXiv 2412.03213: recall at semantic-cluster granularity).
//
// Split-K flash decode: a workgroup takes one chunk of a set's attended rows,
// stages their row sources in LDS (1024 at a time, from the recalled
// positions a previous recall wrote) and streams them through the MFMA
// attention in stream.hpp; the last chunk of a set merges the partials.
#include "stream.hpp"

namespace ckv {

template <int GT>
__global__ __launch_bounds__(kDecThreads) void sparse_decode_kernel(
    const uint16_t* __restrict__ q, int G, const uint16_t* __restrict__ k_tok,
    const uint16_t* __restrict__ v_tok, int capacity, const uint16_t* __restrict__ k_clu,
    const uint16_t* __restrict__ v_clu, int clu_stride, const int32_t* __restrict__ sel_pos,
    const int32_t* __restrict__ sel_count, int budget, int m, int n_sink, int n_clustered,
    int n_total, int chunk_rows, int n_chunks, float* __restrict__ partials, uint32_t* __restrict__ counters,
    float* __restrict__ out, int hs) {
  // ring | row sources; the per-wave merge area reuses both afterwards
  __shared__ __attribute__((aligned(16))) unsigned char smem[kRingBytes + kRowSegment * 4];
  static_assert(kDecWaves * GT * kPartialStride * 4 <= kRingBytes + kRowSegment * 4,
                "merge area must fit in the ring and row sources");
  int* rowsrc = reinterpret_cast<int*>(smem + kRingBytes);

  // attention set u (its queries, recalled positions, partials and output) of
  // physical unit up = u / hs: hs = 1 (one set per KV head shared by its G
  // query heads) or hs = G (one set per query head, G passed as 1)
  const int u = blockIdx.x / n_chunks;
  const int up = u / hs;
  const int c = blockIdx.x % n_chunks;
  const int tid = threadIdx.x;

  StreamState st;
  stream_init(st, q, u, G);
  int cnt = sel_count[u];
  const int cmax = budget < m ? budget : m;
  // Row range of this chunk, bounded without sel_count so that the recalled
  // positions can be fetched while sel_count is still in flight.
  const int R_max = n_sink + cmax + (n_total - n_clustered);
  const int r0 = c * chunk_rows;
  const int r1_max = min(R_max, r0 + chunk_rows);

  RowBases rb;
  rb.ktu = k_tok + (size_t)up * capacity * kHeadDim;
  rb.vtu = v_tok + (size_t)up * capacity * kHeadDim;
  rb.kcu = k_clu + (size_t)up * clu_stride * kHeadDim;
  rb.vcu = v_clu + (size_t)up * clu_stride * kHeadDim;
  rb.knu = rb.ktu;
  rb.vnu = rb.vtu;
  const int32_t* sp = sel_pos + (size_t)u * budget;
  constexpr int kSegPerThread = kRowSegment / kDecThreads;

  for (int seg = r0; seg < r1_max; seg += kRowSegment) {
    const int seg_len_max = min(r1_max, seg + kRowSegment) - seg;
    // recalled positions this thread may need (clamped into sel_pos[u, 0:budget))
    int pos[kSegPerThread];
#pragma unroll
    for (int k = 0; k < kSegPerThread; ++k) {
      const int r = seg + tid + k * kDecThreads;
      const int pi = min(max(r - n_sink, 0), cmax - 1);
      pos[k] = cmax > 0 ? sp[pi] : 0;
    }
    cnt = cnt < 0 ? 0 : (cnt > cmax ? cmax : cnt);
    const int sel_end = n_sink + cnt;
    const int R = sel_end + (n_total - n_clustered);
    const int nrows = max(0, min(min(R, r0 + chunk_rows), seg + kRowSegment) - seg);
    // row sources of this segment: row index, flagged when it lives in the cluster copy
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSegPerThread; ++k) {
      const int i = tid + k * kDecThreads;
      if (i < seg_len_max) {
        const int r = seg + i;
        int v;
        if (r < n_sink) {
          v = r;
        } else if (r < sel_end) {
          const int p = pos[k] < 0 ? 0 : (pos[k] >= m ? m - 1 : pos[k]);
          v = p | kCluFlag;
        } else {
          v = r < R ? n_clustered + (r - sel_end) : 0;
        }
        rowsrc[i] = v;
      }
    }
    __syncthreads();
    stream_rows(st, rb, lds_addr(rowsrc), lds_addr(smem), nrows, G);
  }
  __shared__ int sh_last;
  finish_chunk<GT>(st, reinterpret_cast<float*>(smem), &sh_last, partials, counters, out, u, c, n_chunks, G);
}

static int group_tier(int G) {
  int gt = 1;
  while (gt < G) gt <<= 1;
  return gt;
}

hipError_t launch_sparse_decode(const uint16_t* q, int G, const uint16_t* k_tok,
                                const uint16_t* v_tok, int capacity, const uint16_t* k_clu,
                                const uint16_t* v_clu, int clu_stride, const int32_t* sel_pos,
                                const int32_t* sel_count, int budget, int m, int n_sink,
                                int n_clustered, int n_total, int chunk_rows, int n_chunks,
                                float* partials, uint32_t* counters, float* out, int units, int per_head,
                                hipStream_t s) {
  // per_head: G attention sets per unit, one per query head, each with its own recalled positions
  const int hs = per_head ? G : 1;
  const int Ge = per_head ? 1 : G;
  const dim3 grid((unsigned)(units * hs * n_chunks));
#define CKV_DEC(GTV)                                                                                 \
  hipLaunchKernelGGL(sparse_decode_kernel<GTV>, grid, dim3(kDecThreads), 0, s, q, Ge, k_tok, v_tok, \
                     capacity, k_clu, v_clu, clu_stride, sel_pos, sel_count, budget, m, n_sink,      \
                     n_clustered, n_total, chunk_rows, n_chunks, partials, counters, out, hs)
  switch (group_tier(Ge)) {
    case 1: CKV_DEC(1); break;
    case 2: CKV_DEC(2); break;
    case 4: CKV_DEC(4); break;
    case 8: CKV_DEC(8); break;
    default: CKV_DEC(16); break;
  }
#undef CKV_DEC
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// append: row `row` of every unit's token-order K and V.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void append_kernel(const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new,
                                                    uint16_t* __restrict__ k_tok,
                                                    uint16_t* __restrict__ v_tok, int capacity,
                                                    int row) {
  const int u = blockIdx.x;
  const int lane = threadIdx.x;
  const int part = lane & 15;
  const uint16_t* src = (lane < 16 ? k_new : v_new) + (size_t)u * kHeadDim + part * 8;
  uint16_t* dst = (lane < 16 ? k_tok : v_tok) + ((size_t)u * capacity + row) * kHeadDim + part * 8;
  if (lane < 32) *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}

hipError_t launch_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_tok,
                         uint16_t* v_tok, int capacity, int row, int units, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)units), dim3(64), 0, s, k_new, v_new, k_tok, v_tok,
                     capacity, row);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, size_t n16,
                                                   unsigned char* __restrict__ tail, int ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes - n16 * 16);
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p, n16,
                     (unsigned char*)p + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace ckv
