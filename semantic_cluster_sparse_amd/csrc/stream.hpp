// The streaming half of the flash decode, shared by the decode kernel and the
// fused recall + decode kernel: attention of the query heads of one attended
// set over rows staged as a list of row sources in LDS (ClusterKV article,
// "大模型KV Cache压缩技术：ClusterKV的语义空间优化", §3.1 attention formula;
// §4.1 cluster-contiguous storage), and the split-K merge of the chunks.
//
// A workgroup (8 waves, two per SIMD) streams its rows in tiles of 16.  Each
// wave DMAs its tiles (16 K rows, then 16 V rows, 8 KB) straight from HBM into
// its own LDS ring with global_load_lds_dwordx4, up to kSlots tiles ahead of
// the math, with an XOR swizzle of the 16-byte chunks of every row so that both
// MFMA operand reads are free of bank conflicts.  Per tile:
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
// of a set to finish merges them (log-sum-exp) and writes the normalised
// output.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace ckv {

#ifndef CKV_DEC_SLOTS
#define CKV_DEC_SLOTS 2
#endif
constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kSlots = CKV_DEC_SLOTS;          // tiles per wave ring (kSlots - 1 in flight)
constexpr int kTileBytes = 8192;               // 16 K rows then 16 V rows, 256 B each
constexpr int kRingBytes = kDecWaves * kSlots * kTileBytes;
constexpr int kRowSegment = 1024;              // row sources staged in LDS per segment
// A row source is a row index with a flag for the buffer it lives in:
// token-order cache (no flag), cluster-ordered copy, or the row of the token
// being appended by the same launch (read from the caller's k_new / v_new).
constexpr int kCluFlag = 0x40000000;
constexpr int kNewFlag = 0x20000000;
constexpr int kRowMask = kNewFlag - 1;
static_assert(kSlots >= 2 && 8 * (kSlots - 1) <= 63, "ring depth");
constexpr float kLazy = 8.0f;                  // log2-domain slack before the reference max moves
// Cache policy of the row DMA: non-temporal (each K/V row is read once per
// step), so the stream does not evict the lines that are read again -- the
// centroids, offsets and queries of the recall.  Measured: 29.4 -> 26.9 us per
// fused launch on the 32-layer Llama stack.
constexpr int kStreamPolicy = 2;  // the nt bit of the gfx940-family cache policy

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

// Where the rows of one attended set live: token-order K/V of its unit, the
// cluster-ordered copy, and the appended token's row (may be null).
struct RowBases {
  const uint16_t* ktu;
  const uint16_t* vtu;
  const uint16_t* kcu;
  const uint16_t* vcu;
  const uint16_t* knu;
  const uint16_t* vnu;
};

// Per-lane state of one workgroup's attention stream.
struct StreamState {
  bf16x8 qb[4];     // B operand of S = K Q^T: head hl, head-dim block 32 kb + 8 g .. +7
  float M, lsum;    // reference max (the same in the 4 lanes of a head) and row sum
  f32x4 o[8];       // O[hl][16 nb + 4 g + j]
};

// Queries of set u (G heads, bf16 [sets, G, 128]) into the MFMA B layout and
// an empty accumulator.
__device__ __forceinline__ void stream_init(StreamState& st, const uint16_t* q, int u, int G) {
  const int lane = lane_id();
  const int hl = lane & 15;
  const int g = lane >> 4;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint4 w = hl < G ? *reinterpret_cast<const uint4*>(q + ((size_t)u * G + hl) * kHeadDim + kb * 32 + g * 8)
                           : make_uint4(0, 0, 0, 0);
    st.qb[kb] = __builtin_bit_cast(bf16x8, w);
  }
  st.M = -INFINITY;
  st.lsum = 0.f;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) st.o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Attend to the nrows rows whose sources are staged in LDS at rows_lds (an
// int per row, see kCluFlag / kNewFlag).  Every wave of the workgroup calls
// it; wave w takes tiles w, w + 8, ...  The ring at ring_all (kRingBytes of
// LDS) must be free on entry and is free again on return (every DMA issued is
// waited for).
__device__ __forceinline__ void stream_rows(StreamState& st, const RowBases& rb, uint32_t rows_lds,
                                            uint32_t ring_all, int nrows, int G) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int hl = lane & 15;
  const int g = lane >> 4;
  // DMA lane mapping: op i of a tile covers rows 4i..4i+3; this lane fills
  // chunk slot (lane & 15) of row 4i + (lane >> 4), i.e. global chunk slot ^ swz(row)
  const int dma_slot = lane & 15;
  const uint32_t ring_base = ring_all + (uint32_t)(wave * kSlots * kTileBytes);
  const float qscale = 0.12751743074602468f;  // log2(e) / sqrt(128): scores in the log2 domain
  // per-lane operand offsets inside a tile slot
  uint32_t offk[4], offv[8];
  {
    const int fn = swz(hl);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) offk[kb] = hl * 256 + 16 * ((4 * kb + g) ^ fn);
    const int nr = 4 * g + (hl >> 2);
    const int fr = swz(nr);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      offv[nb] = 4096 + nr * 256 + 16 * ((2 * nb + ((hl & 3) >> 1)) ^ fr) + 8 * (hl & 1);
  }

  // tiles of 16 rows; this wave takes tiles wave, wave + kDecWaves, ...
  const int n_tiles = (nrows + 15) >> 4;
  const int n_tw = n_tiles > wave ? (n_tiles - wave + kDecWaves - 1) / kDecWaves : 0;
  // the bases as values (a select between struct fields by address would keep
  // the struct in memory)
  const uint16_t* const ktu = rb.ktu;
  const uint16_t* const vtu = rb.vtu;
  const uint16_t* const kcu = rb.kcu;
  const uint16_t* const vcu = rb.vcu;
  const uint16_t* const knu = rb.knu;
  const uint16_t* const vnu = rb.vnu;
  auto src = [=](int v, bool val) -> const uint16_t* {
    const uint16_t* t = val ? vtu : ktu;
    const uint16_t* c = val ? vcu : kcu;
    const uint16_t* nw = val ? vnu : knu;
    return (v & kCluFlag) ? c : ((v & kNewFlag) ? nw : t);
  };
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
      const int n = 4 * i + g;
      const size_t off = (size_t)(v[i] & kRowMask) * kHeadDim + 8 * (dma_slot ^ swz(n));
      __builtin_amdgcn_global_load_lds((gptr_t)(src(v[i], false) + off), (lptr_t)(uintptr_t)(slot + 1024 * i),
                                       16, 0, kStreamPolicy);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = 4 * i + g;
      const size_t off = (size_t)(v[i] & kRowMask) * kHeadDim + 8 * (dma_slot ^ swz(n));
      __builtin_amdgcn_global_load_lds((gptr_t)(src(v[i], true) + off),
                                       (lptr_t)(uintptr_t)(slot + 4096 + 1024 * i), 16, 0, kStreamPolicy);
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
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[kb]), st.qb[kb], sacc, 0, 0, 0);
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
    if (__ballot(lmax > st.M + kLazy)) {
      float gm = fmaxf(lmax, __shfl_xor(lmax, 16));
      gm = fmaxf(gm, __shfl_xor(gm, 32));
      const float Mn = gm > st.M + kLazy ? gm : st.M;
      const float alpha = Mn == st.M ? 1.f : __builtin_amdgcn_exp2f(st.M - Mn);  // M = -inf -> 0
      st.lsum *= alpha;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) st.o[nb] *= alpha;
      st.M = Mn;
    }
    // M is -inf only while every score of the head is -inf: p = 0 then
    const float ms = st.M == -INFINITY ? 0.f : st.M;
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sv[e] - ms);
      const float p1 = __builtin_amdgcn_exp2f(sv[e + 1] - ms);
      st.lsum += p0 + p1;
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
      st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, phi, st.o[nb], 0, 0, 0);
      st.o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, plo, st.o[nb], 0, 0, 0);
    }
  }
}

// End of a chunk: the workgroup's (max, sum, output) per head over its 8
// waves (through LDS at red, which may alias the ring: every wave must be done
// with the ring when this is called), then either the normalised output
// (n_chunks == 1) or the chunk partial plus the split-K merge by the last
// chunk of set u to arrive.  counters[u] is zero on entry and on exit.
// flag: one int of LDS outside red.  Returns the chunk's arrival rank among
// the set's chunks (n_chunks - 1 for the chunk that merged, and when
// n_chunks == 1), the same in every thread.
template <int GT>
__device__ __forceinline__ int finish_chunk(StreamState& st, float* red, int* flag, float* __restrict__ partials,
                                            uint32_t* __restrict__ counters, float* __restrict__ out, int u, int c,
                                            int n_chunks, int G) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int hl = lane & 15;
  const int g = lane >> 4;
  // this wave's row sums over its 4 row groups; M is already common to them
  float lsum = st.lsum;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // every wave is done with the ring before it becomes the merge area
  if (hl < G) {
    float* rw = red + (wave * GT + hl) * kPartialStride;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) rw[16 * nb + 4 * g + e] = st.o[nb][e];
    if (g == 0) {
      rw[kHeadDim] = st.M;
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
  if (n_chunks == 1) {  // the whole set in one workgroup: normalise directly
    if (tact) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        out[((size_t)u * G + th) * kHeadDim + td + kTph * i] = wL > 0.f ? wO[i] / wL : 0.f;
    }
    return 0;
  }
  // Chunk partial (max, sum, unnormalised output) per head.  Stores and loads
  // of partials and the arrival counter are device-scope (they bypass the
  // per-XCD L2), so the workgroup that merges may run on any XCD; the drain
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
  if (tid == 0) *flag = (int)__hip_atomic_fetch_add(&counters[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int rank = *flag;
  if (rank != n_chunks - 1) return rank;
  // last chunk of the set to arrive: log-sum-exp merge over all chunks
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
  return rank;
}

}  // namespace ckv
