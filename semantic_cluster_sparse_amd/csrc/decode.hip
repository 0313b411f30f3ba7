// Sparse decode: attention of every query head of a GQA group over the
// recalled rows only -- softmax(q K_S^T / sqrt(d)) V_S with S = sinks, the
// recalled clustered rows (cluster-ordered copy) and the recent unclustered
// rows (ClusterKV article, "大模型KV Cache压缩技术：ClusterKV的语义空间优化",
// §3.1 attention formula; §4.1 cluster-contiguous storage; ClusterKV
// abstract, arXiv 2412.03213: recall at semantic-cluster granularity).
//
// Split-K flash decode built as an HBM stream with the arithmetic on MFMA.
// A workgroup (8 waves, two per SIMD) takes one chunk of one unit's attended
// rows, in tiles of 16 rows.  Each wave DMAs its tiles (16 K rows, then 16 V rows,
// 8 KB) straight from HBM into its own LDS ring with global_load_lds_dwordx4,
// up to kSlots tiles ahead of the math, with an XOR swizzle of the 16-byte
// chunks of every row so that both MFMA operand reads below are free of bank
// conflicts.  Per tile:
//   S = K Q^T     4 x v_mfma_f32_16x16x32_bf16 (M = rows, N = query heads,
//                 K = head dim); lane (h + 16 g) gets rows 4g..4g+3 of head h;
//   softmax       in the log2 domain (q scaled by log2(e)/sqrt(128)) with a
//                 lazily moved reference max per head;
//   O^T += V^T P^T  8 d-blocks x v_mfma_f32_16x16x16_bf16 with V^T read by
//                 ds_read_b64_tr_b16 and P in the layout S left it in (the
//                 contraction index k = 4g + j is row 4g + j of the tile), P
//                 split into bf16 high and low parts (two MFMAs) so that it
//                 keeps ~16 significant bits.
// Each chunk leaves (max, sum, unnormalised output) per head; the last chunk
// of a unit to finish merges them (log-sum-exp) and writes the normalised
// output.
#include "common.hpp"
#include "launch.hpp"

namespace ckv {

#ifndef CKV_DEC_SLOTS
#define CKV_DEC_SLOTS 2
#endif
#ifndef CKV_DEC_THREADS
#define CKV_DEC_THREADS 512
#endif
constexpr int kDecThreads = CKV_DEC_THREADS;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kSlots = CKV_DEC_SLOTS;          // tiles per wave ring (kSlots - 1 in flight)
constexpr int kTileBytes = 8192;               // 16 K rows then 16 V rows, 256 B each
constexpr int kRingBytes = kDecWaves * kSlots * kTileBytes;
constexpr int kRowSegment = 1024;              // row sources staged in LDS per segment
constexpr int kCluFlag = 0x40000000;           // row source is the cluster-ordered copy
static_assert(kSlots >= 2 && 8 * (kSlots - 1) <= 63, "ring depth");
constexpr float kLazy = 8.0f;                  // log2-domain slack before the reference max moves

typedef short s16x4 __attribute__((ext_vector_type(4)));

// gfx9 s_waitcnt immediate with only vmcnt constrained.
#define CKV_VMCNT(N) ((((N) & 15) | (((N) >> 4) << 14)) | (7 << 4) | (15 << 8))

// Wait until at most 8 * min(ahead, N) DMA ops (the 8 ops of each of `ahead`
// younger tiles) are still in flight; ahead <= 0 waits for all.  s_waitcnt
// takes an immediate, hence the unrolled chain over the uniform value.
template <int N>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if constexpr (N <= 0) {
    __builtin_amdgcn_s_waitcnt(CKV_VMCNT(0));
  } else {
    if (ahead >= N)
      __builtin_amdgcn_s_waitcnt(CKV_VMCNT(8 * N));
    else
      wait_tiles<N - 1>(ahead);
  }
}

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// XOR swizzle of the 16-byte chunks of tile row n (0..15): chunk c of row n
// lives at chunk slot c ^ swz(n).  swz is a permutation of 0..15 (so the 16
// rows of one chunk column fall in 16 different bank groups) and every 4
// consecutive rows map a chunk pair {2k, 2k+1} to 4 different pairs (so the
// transposed 4-row reads of V are conflict-free too).
__device__ __forceinline__ int swz(int n) { return ((n << 1) | (n >> 3)) & 15; }

// The row sources of the 4 rows this lane DMAs for a tile (one per 4-row
// group), read from LDS without the compiler seeing it (it would otherwise
// wait for the in-flight LDS DMA of other ring slots).
__device__ __forceinline__ void lds_read_rows4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, int& v0,
                                               int& v1, int& v2, int& v3) {
  asm volatile(
      "ds_read_b32 %0, %4\n\t"
      "ds_read_b32 %1, %5\n\t"
      "ds_read_b32 %2, %6\n\t"
      "ds_read_b32 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// MFMA operands of one tile: the 4 K blocks (A of S = K Q^T, 16 B per lane)
// and the 8 transposed V blocks (A of O^T = V^T P^T, 8 B per lane).
__device__ __forceinline__ void lds_read_tile(uint32_t base, const uint32_t (&ok)[4], const uint32_t (&ov)[8],
                                              uint4 (&k)[4], uint2 (&v)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\t"
      "ds_read_b64_tr_b16 %5, %17\n\t"
      "ds_read_b64_tr_b16 %6, %18\n\t"
      "ds_read_b64_tr_b16 %7, %19\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %21\n\t"
      "ds_read_b64_tr_b16 %10, %22\n\t"
      "ds_read_b64_tr_b16 %11, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]),
        "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(base + ok[0]), "v"(base + ok[1]), "v"(base + ok[2]), "v"(base + ok[3]), "v"(base + ov[0]),
        "v"(base + ov[1]), "v"(base + ov[2]), "v"(base + ov[3]), "v"(base + ov[4]), "v"(base + ov[5]),
        "v"(base + ov[6]), "v"(base + ov[7])
      : "memory");
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {  // RNE; x finite
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

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
  float* red = reinterpret_cast<float*>(smem);

  // attention set u (its queries, recalled positions, partials and output) of
  // physical unit up = u / hs: hs = 1 (one set per KV head shared by its G
  // query heads) or hs = G (one set per query head, G passed as 1)
  const int u = blockIdx.x / n_chunks;
  const int up = u / hs;
  const int c = blockIdx.x % n_chunks;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int hl = lane & 15;  // query head of this lane in the MFMA outputs
  const int g = lane >> 4;   // row group: rows 4g..4g+3 of a tile

  // B operand of S = K Q^T: head hl, head-dim block 32 kb + 8 g .. +7
  bf16x8 qb[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint4 w = hl < G ? *reinterpret_cast<const uint4*>(q + ((size_t)u * G + hl) * kHeadDim + kb * 32 + g * 8)
                           : make_uint4(0, 0, 0, 0);
    qb[kb] = __builtin_bit_cast(bf16x8, w);
  }
  int cnt = sel_count[u];
  const int cmax = budget < m ? budget : m;
  // Row range of this chunk, bounded without sel_count so that the recalled
  // positions can be fetched while sel_count is still in flight.
  const int R_max = n_sink + cmax + (n_total - n_clustered);
  const int r0 = c * chunk_rows;
  const int r1_max = min(R_max, r0 + chunk_rows);

  const float qscale = 0.12751743074602468f;  // log2(e) / sqrt(128): scores in the log2 domain
  float M = -INFINITY, lsum = 0.f;  // reference max (the same in the 4 lanes of a head) and row sum
  f32x4 o[8];                       // O[hl][16 nb + 4 g + j]
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* ktu = k_tok + (size_t)up * capacity * kHeadDim;
  const uint16_t* vtu = v_tok + (size_t)up * capacity * kHeadDim;
  const uint16_t* kcu = k_clu + (size_t)up * clu_stride * kHeadDim;
  const uint16_t* vcu = v_clu + (size_t)up * clu_stride * kHeadDim;
  const int32_t* sp = sel_pos + (size_t)u * budget;
  unsigned char* ring = smem + wave * kSlots * kTileBytes;
  const uint32_t ring_base = lds_addr(ring);
  const uint32_t rows_lds = lds_addr(rowsrc);
  constexpr int kSegPerThread = kRowSegment / kDecThreads;

  // per-lane operand offsets inside a tile slot
  uint32_t offk[4], offv[8];
  {
    const int fn = swz(hl);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) offk[kb] = hl * 256 + 16 * ((4 * kb + g) ^ fn);
    const int s = hl;
    const int nr = 4 * g + (s >> 2);
    const int fr = swz(nr);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      offv[nb] = 4096 + nr * 256 + 16 * ((2 * nb + ((s & 3) >> 1)) ^ fr) + 8 * (s & 1);
  }
  // DMA lane mapping: op i of a tile covers rows 4i..4i+3; this lane fills
  // chunk slot (lane & 15) of row 4i + (lane >> 4), i.e. global chunk slot ^ swz(row)
  const int dma_slot = lane & 15;

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

    // tiles of 16 rows; this wave takes tiles wave, wave + kDecWaves, ...
    const int n_tiles = (nrows + 15) >> 4;
    const int n_tw = n_tiles > wave ? (n_tiles - wave + kDecWaves - 1) / kDecWaves : 0;
    auto issue = [&](int j) {
      const int trow0 = 16 * (wave + j * kDecWaves);
      const uint32_t slot = ring_base + (uint32_t)((j % kSlots) * kTileBytes);
      int v[4];
      uint32_t ra[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ri = trow0 + 4 * i + g;
        ra[i] = rows_lds + (ri < nrows ? ri : 0) * 4;
      }
      lds_read_rows4(ra[0], ra[1], ra[2], ra[3], v[0], v[1], v[2], v[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool clu = (v[i] & kCluFlag) != 0;
        const int n = 4 * i + g;
        const size_t off = (size_t)(v[i] & (kCluFlag - 1)) * kHeadDim + 8 * (dma_slot ^ swz(n));
        __builtin_amdgcn_global_load_lds((gptr_t)((clu ? kcu : ktu) + off),
                                         (lptr_t)(uintptr_t)(slot + 1024 * i), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool clu = (v[i] & kCluFlag) != 0;
        const int n = 4 * i + g;
        const size_t off = (size_t)(v[i] & (kCluFlag - 1)) * kHeadDim + 8 * (dma_slot ^ swz(n));
        __builtin_amdgcn_global_load_lds((gptr_t)((clu ? vcu : vtu) + off),
                                         (lptr_t)(uintptr_t)(slot + 4096 + 1024 * i), 16, 0, 0);
      }
    };
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
      if (j < n_tw) issue(j);

    for (int j = 0; j < n_tw; ++j) {
      // this tile's 8 DMA ops must have landed; younger tiles may stay in flight
      wait_tiles<kSlots - 1>(n_tw - 1 - j);
      uint4 kop[4];
      uint2 vop[8];
      lds_read_tile(ring_base + (uint32_t)((j % kSlots) * kTileBytes), offk, offv, kop, vop);
      if (j + kSlots < n_tw) issue(j + kSlots);

      // S = K Q^T: lane (hl + 16 g) gets rows 4g..4g+3 of head hl
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[kb]), qb[kb], sacc, 0, 0, 0);
      const int trow = 16 * (wave + j * kDecWaves) + 4 * g;
      float sv[4];
      float lmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = hl < G && trow + e < nrows;
        sv[e] = ok ? sacc[e] * qscale : -INFINITY;
        lmax = fmaxf(lmax, sv[e]);
      }
      // Lazy rescaling: the reference max of a head only moves (and its
      // accumulators are rescaled) when a score exceeds it by more than
      // kLazy log2 units, so p = 2^(s - M) stays <= 2^kLazy.  The new max is
      // taken over the head's 4 lanes, so they keep one reference.
      if (__ballot(lmax > M + kLazy)) {
        float gm = fmaxf(lmax, __shfl_xor(lmax, 16));
        gm = fmaxf(gm, __shfl_xor(gm, 32));
        const float Mn = gm > M + kLazy ? gm : M;
        const float alpha = Mn == M ? 1.f : __builtin_amdgcn_exp2f(M - Mn);  // M = -inf -> 0
        lsum *= alpha;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[nb] *= alpha;
        M = Mn;
      }
      // M is -inf only while every score of the head is -inf: p = 0 then
      const float ms = M == -INFINITY ? 0.f : M;
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(sv[e] - ms);
        const float p1 = __builtin_amdgcn_exp2f(sv[e + 1] - ms);
        lsum += p0 + p1;
        const uint32_t h0 = f32_to_bf16_bits(p0), h1 = f32_to_bf16_bits(p1);
        const uint32_t l0 = f32_to_bf16_bits(p0 - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16_bits(p1 - __uint_as_float(h1 << 16));
        hi[e >> 1] = h0 | (h1 << 16);
        lo[e >> 1] = l0 | (l1 << 16);
      }
      const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(hi[0], hi[1]));
      const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(lo[0], lo[1]));
      // O^T += V^T P^T, contraction over the tile's rows (k = 4g + j)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const s16x4 vt = __builtin_bit_cast(s16x4, vop[nb]);
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, phi, o[nb], 0, 0, 0);
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, plo, o[nb], 0, 0, 0);
      }
    }
  }

  // this wave's row sums over its 4 row groups; M is already common to them
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // every wave is done with the ring before it becomes the merge area
  if (hl < G) {
    float* rw = red + (wave * GT + hl) * kPartialStride;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) rw[16 * nb + 4 * g + e] = o[nb][e];
    if (g == 0) {
      rw[kHeadDim] = M;
      rw[kHeadDim + 1] = lsum;
    }
  }
  __syncthreads();
  // Each thread owns kPer head-dim entries of one head, kTph apart (kTph
  // threads per head), so a head's (max, sum) is read once per thread, every
  // load instruction covers contiguous floats, and all of a thread's loads of
  // a merge step are in flight together.
  constexpr int kPer = GT * kHeadDim >= kDecThreads ? GT * kHeadDim / kDecThreads : 1;
  constexpr int kTph = kHeadDim / kPer;
  static_assert(kHeadDim % kPer == 0, "a thread's entries stay inside one head");
  const int th = tid / kTph;  // head of this thread
  const int td = tid % kTph;  // its entries are td + kTph * i
  const bool tact = th < G;
  // this workgroup's (max, sum, unnormalised output) of head th over its 8 waves
  float wM = -INFINITY, wL = 0.f, wO[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) wO[i] = 0.f;
  if (tact) {
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) wM = fmaxf(wM, red[(w * GT + th) * kPartialStride + kHeadDim]);
    const float Ms = (wM == -INFINITY) ? 0.f : wM;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float* rw = red + (w * GT + th) * kPartialStride;
      const float a = exp2f(rw[kHeadDim] - Ms);
      wL += rw[kHeadDim + 1] * a;
#pragma unroll
      for (int i = 0; i < kPer; ++i) wO[i] += rw[td + kTph * i] * a;
    }
  }
  if (n_chunks == 1) {  // the whole unit in one workgroup: normalise directly
    if (tact) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        out[((size_t)u * G + th) * kHeadDim + td + kTph * i] = wL > 0.f ? wO[i] / wL : 0.f;
    }
    return;
  }
  // Chunk partial (max, sum, unnormalised output) per head.  Stores and loads
  // of partials and the arrival counter are device-scope (they bypass the
  // per-XCD L2), so the workgroup that merges may run on any XCD; the wait
  // before the counter increment makes this chunk's stores complete first.
  const size_t cs = (size_t)GT * kPartialStride;
  if (tact) {
    float* outp = partials + ((size_t)u * n_chunks + c) * cs + th * kPartialStride;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      __hip_atomic_store(&outp[td + kTph * i], wO[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (td == 0) {
      __hip_atomic_store(&outp[kHeadDim], wM, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&outp[kHeadDim + 1], wL, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  drain_memory_ops();
  __syncthreads();
  __shared__ int sh_last;
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&counters[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = prev == (uint32_t)(n_chunks - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!sh_last) return;
  // last chunk of the unit to arrive: log-sum-exp merge over all chunks
  if (tact) {
    const float* ph = partials + (size_t)u * n_chunks * cs + th * kPartialStride;
    float M = -INFINITY, L = 0.f, O[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) O[i] = 0.f;
    for (int c0 = 0; c0 < n_chunks; c0 += 8) {
      // all loads of 8 chunks in flight together (indices clamped, extras ignored)
      float mc[8], lc[8], oc[8][kPer];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float* pc = ph + min(c0 + k, n_chunks - 1) * cs;
        mc[k] = __hip_atomic_load(pc + kHeadDim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lc[k] = __hip_atomic_load(pc + kHeadDim + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          oc[k][i] = __hip_atomic_load(pc + td + kTph * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (c0 + k < n_chunks) {
          const float Mn = fmaxf(M, mc[k]);
          const float Ms = (Mn == -INFINITY) ? 0.f : Mn;
          const float a0 = exp2f(M - Ms), a1 = exp2f(mc[k] - Ms);
          L = L * a0 + lc[k] * a1;
#pragma unroll
          for (int i = 0; i < kPer; ++i) O[i] = O[i] * a0 + oc[k][i] * a1;
          M = Mn;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      out[((size_t)u * G + th) * kHeadDim + td + kTph * i] = L > 0.f ? O[i] / L : 0.f;
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
