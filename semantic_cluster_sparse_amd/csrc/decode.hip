// Sparse decode: attention of every query head of a GQA group over the
// recalled rows only -- softmax(q K_S^T / sqrt(d)) V_S with S = sinks, the
// recalled clustered rows (cluster-ordered copy) and the recent unclustered
// rows (ClusterKV article, "大模型KV Cache压缩技术：ClusterKV的语义空间优化",
// §3.1 attention formula; §4.1 cluster-contiguous storage; ClusterKV
// abstract, arXiv 2412.03213: recall at semantic-cluster granularity).
//
// Split-K flash decode built as an HBM stream.  A workgroup (4 waves) takes
// one chunk of one unit's attended rows.  Each wave streams "stages" of 4
// rows (K and V, 2 KB) straight from HBM into its own LDS ring with
// global_load_lds_dwordx4, kStages stages ahead of the math, so every CU keeps
// ~100 KB of row data in flight without spending VGPRs on it.  A 16-lane group
// owns one row of a stage (8 dims per lane) and reads back exactly the bytes
// its lanes DMA'd.  Scores: bf16 dot2 + DPP row sums, log2 domain (q scaled
// by log2(e)/sqrt(128)); softmax updated once per two stages.  Each chunk
// leaves (max, sum, unnormalised output) per head; the last chunk of a unit
// to finish merges them (log-sum-exp) and writes the normalised output.
#include "common.hpp"
#include "launch.hpp"

namespace ckv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}

#ifndef CKV_DEC_STAGES
#define CKV_DEC_STAGES 8
#endif
constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kStages = CKV_DEC_STAGES;     // ring depth per wave (even)
constexpr int kStageBytes = 2048;           // 4 rows x 256 B of K, then of V
constexpr int kRingBytes = kDecWaves * kStages * kStageBytes;
constexpr int kRowSegment = 1024;           // row sources staged in LDS per segment
constexpr int kCluFlag = 0x40000000;        // row source is the cluster-ordered copy
static_assert(kStages % 2 == 0 && kStages >= 4, "stages are consumed two at a time");
constexpr float kLazy = 8.0f;              // log2-domain slack before the reference max moves

// gfx9 s_waitcnt immediate with only vmcnt constrained.
#define CKV_VMCNT(N) ((((N) & 15) | (((N) >> 4) << 14)) | (7 << 4) | (15 << 8))

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// LDS reads the compiler does not see (so it does not wait for the in-flight
// LDS DMA of other ring stages); each waits for its own result.
__device__ __forceinline__ uint4 lds_read_b128(uint32_t addr) {
  uint4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ int lds_read_b32(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
// The two stages consumed by one step (K and V of each) plus the row sources
// of the two stages issued next, with a single wait.
__device__ __forceinline__ void lds_read_step(uint32_t a0, uint32_t a1, uint32_t r0, uint32_t r1, uint4& k0,
                                              uint4& v0, uint4& k1, uint4& v1, int& s0, int& s1) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:1024\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %7 offset:1024\n\t"
      "ds_read_b32 %4, %8\n\t"
      "ds_read_b32 %5, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k0), "=&v"(v0), "=&v"(k1), "=&v"(v1), "=&v"(s0), "=&v"(s1)
      : "v"(a0), "v"(a1), "v"(r0), "v"(r1)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

template <int GT>
__global__ __launch_bounds__(kDecThreads) void sparse_decode_kernel(
    const uint16_t* __restrict__ q, int G, const uint16_t* __restrict__ k_tok,
    const uint16_t* __restrict__ v_tok, int capacity, const uint16_t* __restrict__ k_clu,
    const uint16_t* __restrict__ v_clu, int clu_stride, const int32_t* __restrict__ sel_pos,
    const int32_t* __restrict__ sel_count, int budget, int m, int n_sink, int n_clustered,
    int n_total, int chunk_rows, int n_chunks, float* __restrict__ partials, uint32_t* __restrict__ counters,
    float* __restrict__ out) {
  // ring | row sources; the per-wave merge area reuses the ring afterwards
  __shared__ __attribute__((aligned(16))) unsigned char smem[kRingBytes + kRowSegment * 4];
  static_assert(kDecWaves * GT * kPartialStride * 4 <= kRingBytes, "merge area must fit in the ring");
  int* rowsrc = reinterpret_cast<int*>(smem + kRingBytes);
  float* red = reinterpret_cast<float*>(smem);

  const int u = blockIdx.x / n_chunks;
  const int c = blockIdx.x % n_chunks;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int li = lane & 15;
  const int grp = lane >> 4;  // row of the stage this lane's group owns

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
  unsigned char* ring = smem + wave * kStages * kStageBytes;
  const uint32_t ring_lane = lds_addr(ring) + lane * 16;
  const uint32_t rows_lds = lds_addr(rowsrc);

  for (int seg = r0; seg < r1; seg += kRowSegment) {
    const int seg_end = min(r1, seg + kRowSegment);
    // row sources of this segment: row index, flagged when it lives in the cluster copy
    __syncthreads();
    for (int i = tid; i < seg_end - seg; i += kDecThreads) {
      const int r = seg + i;
      int v;
      if (r < n_sink) {
        v = r;
      } else if (r < sel_end) {
        int p = sp[r];
        p = p < 0 ? 0 : (p >= m ? m - 1 : p);
        v = p | kCluFlag;
      } else {
        v = n_clustered + (r - sel_end);
      }
      rowsrc[i] = v;
    }
    __syncthreads();

    // this wave's stages: 4 consecutive rows each, waves interleaved
    const int nrows = seg_end - seg;
    const int n_st = (nrows + 4 * kDecWaves - 1) / (4 * kDecWaves);  // stages per wave (upper bound)
    // stage st of this wave covers rows 4 * (st * kDecWaves + wave) .. +3 of the segment;
    // a row index past the segment reads entry 0 (its stage is masked out)
    auto src_slot = [&](int st) -> uint32_t {
      const int ri = 4 * (st * kDecWaves + wave) + grp;
      return rows_lds + (ri < nrows ? ri : 0) * 4;
    };
    auto issue = [&](int v, int slot) {
      const bool clu = (v & kCluFlag) != 0;
      const size_t row = (size_t)(v & (kCluFlag - 1)) * kHeadDim;
      unsigned char* dst = ring + slot * kStageBytes;
      __builtin_amdgcn_global_load_lds((gptr_t)((clu ? kcu : ktu) + row), (lptr_t)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gptr_t)((clu ? vcu : vtu) + row), (lptr_t)(dst + 1024), 16, 0, 0);
    };
#pragma unroll
    for (int st = 0; st < kStages; ++st) issue(lds_read_b32(src_slot(st)), st);

    for (int st = 0; st < n_st; st += 2) {
      const int slot = st % kStages;
      // the two oldest stages (4 DMA ops) must have landed; 2 * (kStages - 2) may stay in flight
      __builtin_amdgcn_s_waitcnt(CKV_VMCNT(2 * (kStages - 2)));
      uint4 kr[2], vr[2];
      int nx0, nx1;
      lds_read_step(ring_lane + slot * kStageBytes, ring_lane + (slot + 1) * kStageBytes,
                    src_slot(st + kStages), src_slot(st + kStages + 1), kr[0], vr[0], kr[1], vr[1], nx0,
                    nx1);
      issue(nx0, slot);
      issue(nx1, slot + 1);

      float s[2][GT];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const bool ok = 4 * ((st + k) * kDecWaves + wave) + grp < nrows;
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
      // Lazy rescaling: the reference max only moves (and the accumulators
      // are rescaled) when a score exceeds it by more than kLazy in log2
      // units, so p = 2^(s - ref) stays <= 2^kLazy; the merge divides it out.
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float mn = fmaxf(s[0][h], s[1][h]);
        if (mn > mx[h] + kLazy) {
          const float alpha = mx[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx[h] - mn);
          ls[h] *= alpha;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
          mx[h] = mn;
        }
        // mx is -inf only while every score seen is -inf (masked rows): p = 0 then
        const float ms = mx[h] == -INFINITY ? 0.f : mx[h];
        const float p0 = __builtin_amdgcn_exp2f(s[0][h] - ms);
        const float p1 = __builtin_amdgcn_exp2f(s[1][h] - ms);
        ls[h] += p0 + p1;
        acc[h][0] = fmaf(p1, bf16_lo(vr[1].x), fmaf(p0, bf16_lo(vr[0].x), acc[h][0]));
        acc[h][1] = fmaf(p1, bf16_hi(vr[1].x), fmaf(p0, bf16_hi(vr[0].x), acc[h][1]));
        acc[h][2] = fmaf(p1, bf16_lo(vr[1].y), fmaf(p0, bf16_lo(vr[0].y), acc[h][2]));
        acc[h][3] = fmaf(p1, bf16_hi(vr[1].y), fmaf(p0, bf16_hi(vr[0].y), acc[h][3]));
        acc[h][4] = fmaf(p1, bf16_lo(vr[1].z), fmaf(p0, bf16_lo(vr[0].z), acc[h][4]));
        acc[h][5] = fmaf(p1, bf16_hi(vr[1].z), fmaf(p0, bf16_hi(vr[0].z), acc[h][5]));
        acc[h][6] = fmaf(p1, bf16_lo(vr[1].w), fmaf(p0, bf16_lo(vr[0].w), acc[h][6]));
        acc[h][7] = fmaf(p1, bf16_hi(vr[1].w), fmaf(p0, bf16_hi(vr[0].w), acc[h][7]));
      }
    }
    // drain the DMA issued past the end of this wave's stages before the ring is reused
    __builtin_amdgcn_s_waitcnt(CKV_VMCNT(0));
  }

  // merge the 4 row groups of this wave (lane bits 4 and 5)
#pragma unroll
  for (int o = 16; o < kWave; o <<= 1) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float mo = __shfl_xor(mx[h], o);
      const float lo = __shfl_xor(ls[h], o);
      const float M = fmaxf(mx[h], mo);
      const float Ms = (M == -INFINITY) ? 0.f : M;
      const float as = exp2f(mx[h] - Ms), ao = exp2f(mo - Ms);
      ls[h] = ls[h] * as + lo * ao;
      mx[h] = M;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float other = __shfl_xor(acc[h][e], o);
        acc[h][e] = acc[h][e] * as + other * ao;
      }
    }
  }
  __syncthreads();  // every wave is done with the ring before it becomes the merge area
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float* rw = red + (wave * GT + h) * kPartialStride;
#pragma unroll
      for (int e = 0; e < 8; ++e) rw[li * 8 + e] = acc[h][e];
      if (lane == 0) {
        rw[kHeadDim] = mx[h];
        rw[kHeadDim + 1] = ls[h];
      }
    }
  }
  __syncthreads();
  if (n_chunks == 1) {  // the whole unit in one workgroup: normalise directly
    for (int t = tid; t < G * kHeadDim; t += kDecThreads) {
      const int h = t / kHeadDim, d = t % kHeadDim;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red[(w * GT + h) * kPartialStride + kHeadDim]);
      const float Ms = (M == -INFINITY) ? 0.f : M;
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float* rw = red + (w * GT + h) * kPartialStride;
        const float a = exp2f(rw[kHeadDim] - Ms);
        L += rw[kHeadDim + 1] * a;
        O += rw[d] * a;
      }
      out[((size_t)u * G + h) * kHeadDim + d] = L > 0.f ? O / L : 0.f;
    }
    return;
  }
  // Chunk partial (max, sum, unnormalised output) per head.  Stores and loads
  // of partials and the arrival counter are device-scope (they bypass the
  // per-XCD L2), so the workgroup that merges may run on any XCD; the wait
  // before the counter increment makes this chunk's stores complete first.
  const size_t cs = (size_t)GT * kPartialStride;
  float* outp = partials + ((size_t)u * n_chunks + c) * cs;
  for (int t = tid; t < G * kHeadDim; t += kDecThreads) {
    const int h = t / kHeadDim, d = t % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red[(w * GT + h) * kPartialStride + kHeadDim]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float* rw = red + (w * GT + h) * kPartialStride;
      const float a = exp2f(rw[kHeadDim] - Ms);
      L += rw[kHeadDim + 1] * a;
      O += rw[d] * a;
    }
    __hip_atomic_store(&outp[h * kPartialStride + d], O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(&outp[h * kPartialStride + kHeadDim], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&outp[h * kPartialStride + kHeadDim + 1], L, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int sh_last;
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&counters[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == (uint32_t)(n_chunks - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;
  // last chunk of the unit to arrive: log-sum-exp merge over all chunks, every load independent
  const float* p = partials + (size_t)u * n_chunks * cs;
  for (int t = tid; t < G * kHeadDim; t += kDecThreads) {
    const int h = t / kHeadDim, d = t % kHeadDim;
    const float* ph = p + h * kPartialStride;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int cc = 0; cc < n_chunks; ++cc) {
      const float mc = __hip_atomic_load(ph + cc * cs + kHeadDim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float lc = __hip_atomic_load(ph + cc * cs + kHeadDim + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float oc = __hip_atomic_load(ph + cc * cs + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

hipError_t launch_sparse_decode(const uint16_t* q, int G, const uint16_t* k_tok,
                                const uint16_t* v_tok, int capacity, const uint16_t* k_clu,
                                const uint16_t* v_clu, int clu_stride, const int32_t* sel_pos,
                                const int32_t* sel_count, int budget, int m, int n_sink,
                                int n_clustered, int n_total, int chunk_rows, int n_chunks,
                                float* partials, uint32_t* counters, float* out, int units, hipStream_t s) {
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
