// Sparse decode: attention of every query head of a GQA group over the
// recalled rows only -- softmax(q K_S^T / sqrt(d)) V_S with S = sinks, the
// recalled clustered rows (cluster-ordered copy) and the recent unclustered
// rows (ClusterKV article, "大模型KV Cache压缩技术：ClusterKV的语义空间优化",
// §3.1 attention formula; §4.1 cluster-contiguous storage; ClusterKV
// abstract, arXiv 2412.03213: recall at semantic-cluster granularity).
//
// Split-K flash decode: a workgroup takes one chunk of the attended rows of
// one unit; LPR lanes share a row (DPL = 128/LPR dims each), every row is
// read once for all G heads; scores live in the log2 domain (q pre-scaled by
// log2(e)/sqrt(128)); each workgroup leaves (max, sum, unnormalised output)
// per head, merged by a small log-sum-exp kernel.
#include "common.hpp"
#include "launch.hpp"

namespace ckv {

template <int DPL>
struct RowPart;
template <>
struct RowPart<8> {
  typedef uint4 T;
  __device__ static __forceinline__ void unpack(const T& w, float* x) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
};
template <>
struct RowPart<4> {
  typedef uint2 T;
  __device__ static __forceinline__ void unpack(const T& w, float* x) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  }
};
template <>
struct RowPart<2> {
  typedef uint32_t T;
  __device__ static __forceinline__ void unpack(const T& w, float* x) {
    x[0] = bf16_lo(w); x[1] = bf16_hi(w);
  }
};

template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void merge_state(float& m, float& l, float mo, float lo, float& a_self,
                                            float& a_other) {
  const float M = fmaxf(m, mo);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  a_self = exp2f(m - Ms);
  a_other = exp2f(mo - Ms);
  l = l * a_self + lo * a_other;
  m = M;
}

constexpr int kDecThreads = 256;

template <int GT, int LPR>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, int G, const uint16_t* __restrict__ k_tok,
    const uint16_t* __restrict__ v_tok, int capacity, const uint16_t* __restrict__ k_clu,
    const uint16_t* __restrict__ v_clu, int clu_stride, const int32_t* __restrict__ sel_pos,
    const int32_t* __restrict__ sel_count, int budget, int m, int n_sink, int n_clustered,
    int n_total, int chunk_rows, int n_chunks, float* __restrict__ partials) {
  constexpr int DPL = kHeadDim / LPR;
  constexpr int NG = kDecThreads / LPR;      // row groups per workgroup
  constexpr int kDecUnroll = (GT >= 8) ? 2 : 4;  // rows in flight per row group
  typedef typename RowPart<DPL>::T PartT;
  __shared__ float red[kDecThreads / kWave][GT][kPartialStride];

  const int u = blockIdx.x / n_chunks;
  const int c = blockIdx.x % n_chunks;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int li = lane % LPR;
  const int gi = tid / LPR;

  int cnt = sel_count[u];
  const int cmax = budget < m ? budget : m;
  cnt = cnt < 0 ? 0 : (cnt > cmax ? cmax : cnt);
  const int R = n_sink + cnt + (n_total - n_clustered);
  const int r0 = c * chunk_rows;
  const int r1 = min(R, r0 + chunk_rows);

  const float qscale = 0.12751743074602468f;  // log2(e) / sqrt(128)
  float qv[GT][DPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    if (h < G) {
      const PartT w = *reinterpret_cast<const PartT*>(q + ((size_t)u * G + h) * kHeadDim + li * DPL);
      RowPart<DPL>::unpack(w, qv[h]);
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[h][e] *= qscale;
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[h][e] = 0.f;
    }
  }

  float mx[GT], ls[GT], acc[GT][DPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    mx[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
  }

  const size_t tok_base = (size_t)u * capacity * kHeadDim;
  const size_t clu_base = (size_t)u * clu_stride * kHeadDim;
  const int32_t* sp = sel_pos + (size_t)u * budget;
  const int sel_end = n_sink + cnt;

  for (int base = r0 + gi; base < r1; base += NG * kDecUnroll) {
    PartT kw[kDecUnroll], vw[kDecUnroll];
    bool ok[kDecUnroll];
#pragma unroll
    for (int k = 0; k < kDecUnroll; ++k) {
      const int r = base + k * NG;
      ok[k] = r < r1;
      size_t off;
      const uint16_t *kb, *vb;
      if (!ok[k] || r < n_sink) {
        off = tok_base + (size_t)(ok[k] ? r : 0) * kHeadDim;
        kb = k_tok;
        vb = v_tok;
      } else if (r < sel_end) {
        int p = sp[r - n_sink];
        p = p < 0 ? 0 : (p >= m ? m - 1 : p);
        off = clu_base + (size_t)p * kHeadDim;
        kb = k_clu;
        vb = v_clu;
      } else {
        off = tok_base + (size_t)(n_clustered + (r - sel_end)) * kHeadDim;
        kb = k_tok;
        vb = v_tok;
      }
      kw[k] = *reinterpret_cast<const PartT*>(kb + off + li * DPL);
      vw[k] = *reinterpret_cast<const PartT*>(vb + off + li * DPL);
    }
    float s[kDecUnroll][GT];
#pragma unroll
    for (int k = 0; k < kDecUnroll; ++k) {
      float x[DPL];
      RowPart<DPL>::unpack(kw[k], x);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) d = fmaf(qv[h][e], x[e], d);
        d = row_sum<LPR>(d);
        s[k][h] = ok[k] ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float mn = mx[h];
#pragma unroll
      for (int k = 0; k < kDecUnroll; ++k) mn = fmaxf(mn, s[k][h]);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = exp2f(mx[h] - ms);
      ls[h] *= alpha;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[h][e] *= alpha;
      mx[h] = mn;
#pragma unroll
      for (int k = 0; k < kDecUnroll; ++k) {
        const float p = exp2f(s[k][h] - ms);
        ls[h] += p;
        float v[DPL];
        RowPart<DPL>::unpack(vw[k], v);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
      }
    }
  }

  // merge the row groups of this wave (lanes differing in the bits above LPR)
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float mo = __shfl_xor(mx[h], o);
      const float lo = __shfl_xor(ls[h], o);
      float as, ao;
      merge_state(mx[h], ls[h], mo, lo, as, ao);
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float other = __shfl_xor(acc[h][e], o);
        acc[h][e] = acc[h][e] * as + other * ao;
      }
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) red[wave][h][li * DPL + e] = acc[h][e];
      if (lane == 0) {
        red[wave][h][kHeadDim] = mx[h];
        red[wave][h][kHeadDim + 1] = ls[h];
      }
    }
  }
  __syncthreads();
  constexpr int NW = kDecThreads / kWave;
  float* outp = partials + ((size_t)u * n_chunks + c) * GT * kPartialStride;
  for (int t = tid; t < GT * kHeadDim; t += kDecThreads) {
    const int h = t / kHeadDim, d = t % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red[w][h][kHeadDim]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = exp2f(red[w][h][kHeadDim] - Ms);
      L += red[w][h][kHeadDim + 1] * a;
      O += red[w][h][d] * a;
    }
    outp[h * kPartialStride + d] = O;
    if (d == 0) {
      outp[h * kPartialStride + kHeadDim] = M;
      outp[h * kPartialStride + kHeadDim + 1] = L;
    }
  }
}

// One workgroup of 128 threads per (unit, head): log-sum-exp merge of the chunks.
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ partials,
                                                             int GT, int G, int n_chunks,
                                                             float* __restrict__ out) {
  const int u = blockIdx.x / G;
  const int h = blockIdx.x % G;
  const int d = threadIdx.x;
  const float* p = partials + (size_t)u * n_chunks * GT * kPartialStride + h * kPartialStride;
  const size_t cs = (size_t)GT * kPartialStride;
  float M = -INFINITY;
  for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, p[c * cs + kHeadDim]);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  float L = 0.f, O = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    const float a = exp2f(p[c * cs + kHeadDim] - Ms);
    L += p[c * cs + kHeadDim + 1] * a;
    O += p[c * cs + d] * a;
  }
  out[((size_t)u * G + h) * kHeadDim + d] = L > 0.f ? O / L : 0.f;
}

template <int GT, int LPR>
static void launch_split(dim3 grid, hipStream_t s, const uint16_t* q, int G, const uint16_t* k_tok,
                         const uint16_t* v_tok, int capacity, const uint16_t* k_clu,
                         const uint16_t* v_clu, int clu_stride, const int32_t* sel_pos,
                         const int32_t* sel_count, int budget, int m, int n_sink, int n_clustered,
                         int n_total, int chunk_rows, int n_chunks, float* partials) {
  hipLaunchKernelGGL((decode_split_kernel<GT, LPR>), grid, dim3(kDecThreads), 0, s, q, G, k_tok,
                     v_tok, capacity, k_clu, v_clu, clu_stride, sel_pos, sel_count, budget, m,
                     n_sink, n_clustered, n_total, chunk_rows, n_chunks, partials);
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
                                float* partials, float* out, int units, hipStream_t s) {
  const dim3 grid((unsigned)(units * n_chunks));
  const int gt = group_tier(G);
#define CKV_SPLIT(GTV, LPRV)                                                                      \
  launch_split<GTV, LPRV>(grid, s, q, G, k_tok, v_tok, capacity, k_clu, v_clu, clu_stride,       \
                          sel_pos, sel_count, budget, m, n_sink, n_clustered, n_total, chunk_rows, \
                          n_chunks, partials)
  switch (gt) {
    case 1: CKV_SPLIT(1, 16); break;
    case 2: CKV_SPLIT(2, 16); break;
    case 4: CKV_SPLIT(4, 16); break;
    case 8: CKV_SPLIT(8, 32); break;
    default: CKV_SPLIT(16, 32); break;
  }
#undef CKV_SPLIT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(units * G)), dim3(128), 0, s, partials, gt,
                     G, n_chunks, out);
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
