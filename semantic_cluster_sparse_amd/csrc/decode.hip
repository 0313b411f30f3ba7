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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

constexpr int kDecThreads = 256;
constexpr int kDecGroups = kDecThreads / 16;  // row groups of 16 lanes (8 dims per lane)

// Rows per row group per batch: all are loaded before any arithmetic.
template <int GT>
struct DecRows {
  static constexpr int U = GT <= 4 ? 8 : (GT == 8 ? 4 : 2);
};

__device__ __forceinline__ void merge_state(float& m, float& l, float mo, float lo, float& a_self,
                                            float& a_other) {
  const float M = fmaxf(m, mo);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  a_self = exp2f(m - Ms);
  a_other = exp2f(mo - Ms);
  l = l * a_self + lo * a_other;
  m = M;
}

// One workgroup per (unit, chunk of attended rows).  Row r of the attended
// sequence is a sink (r < n_sink), a recalled row of the cluster-ordered copy
// (r < n_sink + cnt, position sel_pos[r - n_sink]) or a recent row.  Each
// workgroup leaves per head (max, sum, unnormalised output) in `partials`;
// the last workgroup of the unit to finish (arrival counter in `counters`,
// reset to 0 by that workgroup) merges them into `out`.
template <int GT>
__global__ __launch_bounds__(kDecThreads) void sparse_decode_kernel(
    const uint16_t* __restrict__ q, int G, const uint16_t* __restrict__ k_tok,
    const uint16_t* __restrict__ v_tok, int capacity, const uint16_t* __restrict__ k_clu,
    const uint16_t* __restrict__ v_clu, int clu_stride, const int32_t* __restrict__ sel_pos,
    const int32_t* __restrict__ sel_count, int budget, int m, int n_sink, int n_clustered,
    int n_total, int chunk_rows, int n_chunks, float* __restrict__ partials,
    uint32_t* __restrict__ counters, float* __restrict__ out) {
  constexpr int U = DecRows<GT>::U;
  constexpr int NW = kDecThreads / kWave;
  __shared__ float red[NW][GT][kPartialStride];
  __shared__ int sh_last;
  __shared__ int rowsrc[kDecGroups * DecRows<GT>::U];

  const int u = blockIdx.x / n_chunks;
  const int c = blockIdx.x % n_chunks;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int li = tid & 15;
  const int gi = tid >> 4;

  uint4 qw[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h)
    qw[h] = h < G ? *reinterpret_cast<const uint4*>(q + ((size_t)u * G + h) * kHeadDim + li * 8)
                  : make_uint4(0, 0, 0, 0);

  int cnt = sel_count[u];
  const int cmax = budget < m ? budget : m;
  cnt = cnt < 0 ? 0 : (cnt > cmax ? cmax : cnt);
  const int sel_end = n_sink + cnt;
  const int R = sel_end + (n_total - n_clustered);
  const int r0 = c * chunk_rows;
  const int r1 = min(R, r0 + chunk_rows);

  const float qscale = 0.12751743074602468f;  // log2(e) / sqrt(128): scores in the log2 domain
  float mx[GT], ls[GT], acc[GT][8];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    mx[h] = -INFINITY;
    ls[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const uint16_t* ktu = k_tok + (size_t)u * capacity * kHeadDim + li * 8;
  const uint16_t* vtu = v_tok + (size_t)u * capacity * kHeadDim + li * 8;
  const uint16_t* kcu = k_clu + (size_t)u * clu_stride * kHeadDim + li * 8;
  const uint16_t* vcu = v_clu + (size_t)u * clu_stride * kHeadDim + li * 8;
  const int32_t* sp = sel_pos + (size_t)u * budget - n_sink;

  // Rows of a batch are staged as source indices in LDS (one coalesced load of
  // sel_pos per batch), so every row load of the batch issues back to back.
  constexpr int kBatch = kDecGroups * U;
  constexpr int kCluFlag = 0x40000000;
  for (int bs = r0; bs < r1; bs += kBatch) {
    if (tid < kBatch) {
      const int r = bs + tid;
      int v = 0;
      if (r < r1) {
        if (r < n_sink) {
          v = r;
        } else if (r < sel_end) {
          int p = sp[r];
          p = p < 0 ? 0 : (p >= m ? m - 1 : p);
          v = p | kCluFlag;
        } else {
          v = n_clustered + (r - sel_end);
        }
      }
      rowsrc[tid] = v;
    }
    __syncthreads();
    uint4 kr[U], vr[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int v = rowsrc[gi + k * kDecGroups];
      const bool clu = (v & kCluFlag) != 0;
      const size_t row = (size_t)(v & (kCluFlag - 1)) * kHeadDim;
      kr[k] = *reinterpret_cast<const uint4*>((clu ? kcu : ktu) + row);
      vr[k] = *reinterpret_cast<const uint4*>((clu ? vcu : vtu) + row);
    }
    __syncthreads();
    // keep the scheduler from interleaving math between the row loads
    __builtin_amdgcn_sched_barrier(0);
    const int b0 = bs + gi;
    float s[U][GT];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const bool ok = b0 + k * kDecGroups < r1;
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float d = dot2(kr[k].x, qw[h].x, 0.f);
        d = dot2(kr[k].y, qw[h].y, d);
        d = dot2(kr[k].z, qw[h].z, d);
        d = dot2(kr[k].w, qw[h].w, d);
        d = sum16(d);
        s[k][h] = ok ? d * qscale : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float mn = mx[h];
#pragma unroll
      for (int k = 0; k < U; ++k) mn = fmaxf(mn, s[k][h]);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = exp2f(mx[h] - ms);
      ls[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      mx[h] = mn;
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const float p = exp2f(s[k][h] - ms);
        ls[h] += p;
        acc[h][0] = fmaf(p, bf16_lo(vr[k].x), acc[h][0]);
        acc[h][1] = fmaf(p, bf16_hi(vr[k].x), acc[h][1]);
        acc[h][2] = fmaf(p, bf16_lo(vr[k].y), acc[h][2]);
        acc[h][3] = fmaf(p, bf16_hi(vr[k].y), acc[h][3]);
        acc[h][4] = fmaf(p, bf16_lo(vr[k].z), acc[h][4]);
        acc[h][5] = fmaf(p, bf16_hi(vr[k].z), acc[h][5]);
        acc[h][6] = fmaf(p, bf16_lo(vr[k].w), acc[h][6]);
        acc[h][7] = fmaf(p, bf16_hi(vr[k].w), acc[h][7]);
      }
    }
  }

  // merge the 4 row groups of this wave (lane bits 4 and 5)
#pragma unroll
  for (int o = 16; o < kWave; o <<= 1) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float mo = __shfl_xor(mx[h], o);
      const float lo = __shfl_xor(ls[h], o);
      float as, ao;
      merge_state(mx[h], ls[h], mo, lo, as, ao);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float other = __shfl_xor(acc[h][e], o);
        acc[h][e] = acc[h][e] * as + other * ao;
      }
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][h][li * 8 + e] = acc[h][e];
      if (lane == 0) {
        red[wave][h][kHeadDim] = mx[h];
        red[wave][h][kHeadDim + 1] = ls[h];
      }
    }
  }
  __syncthreads();
  float* pu = partials + (size_t)u * n_chunks * GT * kPartialStride;
  float* outp = pu + (size_t)c * GT * kPartialStride;
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
    // device-scope stores: written through to the coherence point shared by all
    // XCDs, so the merging workgroup sees them without a cache-wide flush
    __hip_atomic_store(&outp[h * kPartialStride + d], O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(&outp[h * kPartialStride + kHeadDim], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&outp[h * kPartialStride + kHeadDim + 1], L, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // Arrival: every thread waits until its device-scope partial stores are
  // acknowledged (vmcnt covers stores on gfx9), then the barrier, then one
  // relaxed device-scope increment; the last chunk of the unit merges.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&counters[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = (prev == (uint32_t)(n_chunks - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;
  const size_t cs = (size_t)GT * kPartialStride;
  for (int t = tid; t < G * kHeadDim; t += kDecThreads) {
    const int h = t / kHeadDim, d = t % kHeadDim;
    const float* p = pu + h * kPartialStride;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int cc = 0; cc < n_chunks; ++cc) {  // online merge: one pass over the chunks
      const float mc = __hip_atomic_load(p + cc * cs + kHeadDim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float lc = __hip_atomic_load(p + cc * cs + kHeadDim + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float oc = __hip_atomic_load(p + cc * cs + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float Mn = fmaxf(M, mc);
      const float Ms = (Mn == -INFINITY) ? 0.f : Mn;
      const float a0 = exp2f(M - Ms), a1 = exp2f(mc - Ms);
      L = L * a0 + lc * a1;
      O = O * a0 + oc * a1;
      M = Mn;
    }
    out[((size_t)u * G + h) * kHeadDim + d] = L > 0.f ? O / L : 0.f;
  }
  if (tid == 0) __hip_atomic_store(&counters[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static int group_tier(int G) {
  int gt = 1;
  while (gt < G) gt <<= 1;
  return gt;
}

int decode_rows_per_batch(int G) {
  switch (group_tier(G)) {
    case 1: return kDecGroups * DecRows<1>::U;
    case 2: return kDecGroups * DecRows<2>::U;
    case 4: return kDecGroups * DecRows<4>::U;
    case 8: return kDecGroups * DecRows<8>::U;
    default: return kDecGroups * DecRows<16>::U;
  }
}

hipError_t launch_sparse_decode(const uint16_t* q, int G, const uint16_t* k_tok,
                                const uint16_t* v_tok, int capacity, const uint16_t* k_clu,
                                const uint16_t* v_clu, int clu_stride, const int32_t* sel_pos,
                                const int32_t* sel_count, int budget, int m, int n_sink,
                                int n_clustered, int n_total, int chunk_rows, int n_chunks,
                                float* partials, uint32_t* counters, float* out, int units,
                                hipStream_t s) {
  const dim3 grid((unsigned)(units * n_chunks));
#define CKV_DEC(GTV)                                                                                \
  hipLaunchKernelGGL(sparse_decode_kernel<GTV>, grid, dim3(kDecThreads), 0, s, q, G, k_tok, v_tok, \
                     capacity, k_clu, v_clu, clu_stride, sel_pos, sel_count, budget, m, n_sink,     \
                     n_clustered, n_total, chunk_rows, n_chunks, partials, counters, out)
  switch (group_tier(G)) {
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
