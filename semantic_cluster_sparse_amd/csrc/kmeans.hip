// Cosine K-means kernels: initial directions, MFMA assignment with a fused
// row argmax, a one-launch stable counting sort by label, and the
// per-cluster segmented reduction that updates the centroid state and writes
// the cluster-contiguous copy of the K/V rows.
//
// Method: ClusterKV article ("大模型KV Cache压缩技术：ClusterKV的语义空间优化"),
// §3.2 (cosine K-means over the non-sink keys at prefill; online incremental
// clustering during decoding), §3.1 (the centroid as the members' mean),
// §4.1 (half-precision matrix multiply for the distances; cluster-contiguous
// KV storage).
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace ckv {

// ---------------------------------------------------------------------------
// Seeded initial indices (the prefill's initialisation, which the ClusterKV
// article leaves open): K distinct clustered-token indices per unit drawn by
// Floyd's sampling algorithm (Bentley and Floyd, CACM 1987) from SplitMix64
// outputs (Steele, Lea and Flood, OOPSLA 2014), state seed + unit.  For
// j = m - K .. m - 1 a draw r gives t = r mod (j + 1); t is inserted unless it
// is already in the sample, in which case j is.  One workgroup per unit.  The
// generator's state after i + 1 steps is its initial state plus (i + 1) times
// its increment, so the lanes compute every draw's t at once.
// ---------------------------------------------------------------------------
constexpr uint64_t kSplitMixGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// t of every draw of unit u into t_out[0, K)
__device__ __forceinline__ void floyd_targets(uint64_t seed, int u, int m, int K, int* t_out) {
  const uint64_t s0 = seed + (uint64_t)u;
  for (int i = lane_id(); i < K; i += kWave) {
    const uint64_t r = splitmix64_mix(s0 + (uint64_t)(i + 1) * kSplitMixGamma);
    t_out[i] = (int)(r % (uint64_t)(m - K + i + 1));
  }
}

// Membership of the indices drawn so far: a bitmap over [0, m) in LDS when it
// fits, else the list of draws scanned by all 64 lanes.
constexpr int kDrawBitmapWords = 16384;  // 64 KiB of LDS: m up to 524288

// The bitmap form takes the draws 64 at a time, one per lane.  With low = m - K,
// draw i's target t lies in [0, low + i], and t is already in the sample when
// (a) an earlier batch inserted it (the bitmap), (b) an earlier draw of this
// batch has the same target (that draw inserted t, or t was in already), or
// (c) t = low + j for an earlier draw j of this batch that found its own target
// taken and so inserted low + j.  (c) links a draw to one earlier draw; the
// links are resolved by repeating it until no flag changes (each repetition
// settles at least one more link of every chain, so at most 64 repetitions).
// The result equals inserting the draws one after another.
__global__ __launch_bounds__(64) void init_draw_bitmap_kernel(uint64_t seed, int m, int K,
                                                              int32_t* __restrict__ init_idx) {
  extern __shared__ uint32_t bitmap[];
  const int u = blockIdx.x;
  const int lane = lane_id();
  const int words = (m + 31) >> 5;
  for (int i = lane; i < words; i += kWave) bitmap[i] = 0u;
  __syncthreads();
  const uint64_t s0 = seed + (uint64_t)u;
  const int low = m - K;
  int32_t* out = init_idx + (size_t)u * K;
  for (int base = 0; base < K; base += kWave) {
    const int i = base + lane;
    const bool live = i < K;
    int t = 0;
    if (live) {
      const uint64_t r = splitmix64_mix(s0 + (uint64_t)(i + 1) * kSplitMixGamma);
      t = (int)(r % (uint64_t)(low + i + 1));
    }
    bool taken = (bitmap[t >> 5] >> (t & 31)) & 1u;
#pragma unroll 8
    for (int j = 0; j < kWave - 1; ++j) taken |= (j < lane) & (__builtin_amdgcn_readlane(t, j) == t);
    taken = taken && live;
    const int src = t - low - base;  // lane of the draw whose own index is t
    const bool linked = live && src >= 0 && src < lane;
    unsigned long long cur = __ballot(taken), prev = 0;
    while (cur != prev) {
      prev = cur;
      taken = taken || (linked && ((cur >> (src & 63)) & 1ull));
      cur = __ballot(taken);
    }
    const int pick = taken ? low + i : t;  // low + i itself is never taken: every earlier pick is below it
    if (live) {
      atomicOr(&bitmap[pick >> 5], 1u << (pick & 31));
      out[i] = pick;
    }
    __syncthreads();  // the inserts are seen by the next batch's membership tests
  }
}

__global__ __launch_bounds__(64) void init_draw_kernel(uint64_t seed, int m, int K, int32_t* __restrict__ init_idx) {
  __shared__ int chosen[kMaxClusters];
  __shared__ int tdraw[kMaxClusters];
  const int u = blockIdx.x;
  const int lane = lane_id();
  floyd_targets(seed, u, m, K, tdraw);
  __syncthreads();
  for (int i = 0; i < K; ++i) {
    const int t = tdraw[i];
    bool hit = false;
    for (int c = lane; c < i; c += kWave) hit |= chosen[c] == t;
    const int pick = __ballot(hit) ? m - K + i : t;
    if (lane == 0) chosen[i] = pick;
    __syncthreads();  // the insert is seen by every lane's next membership test
  }
  for (int i = lane; i < K; i += kWave) init_idx[(size_t)u * K + i] = chosen[i];
}

hipError_t launch_init_draw(uint64_t seed, int m, int K, int32_t* init_idx, int units, hipStream_t s) {
  const int words = (m + 31) / 32;
  if (words <= kDrawBitmapWords) {
    static std::once_flag lds_attr;  // the bitmap may exceed the default dynamic LDS limit
    static hipError_t lds_err = hipSuccess;
    std::call_once(lds_attr, [] {
      lds_err = hipFuncSetAttribute((const void*)init_draw_bitmap_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    kDrawBitmapWords * 4);
    });
    if (lds_err != hipSuccess) return lds_err;
    hipLaunchKernelGGL(init_draw_bitmap_kernel, dim3((unsigned)units), dim3(kWave), (size_t)words * 4, s, seed, m, K,
                       init_idx);
  } else {
    hipLaunchKernelGGL(init_draw_kernel, dim3((unsigned)units), dim3(kWave), 0, s, seed, m, K, init_idx);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Initial directions: one wave per (unit, cluster); lane l holds dims 2l, 2l+1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void init_dirs_kernel(const uint16_t* __restrict__ k_tok,
                                                        int capacity, int n_sink, int m,
                                                        const int32_t* __restrict__ init_idx,
                                                        int K, uint16_t* __restrict__ cdir,
                                                        int units) {
  const int lane = lane_id();
  const long gw = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= (long)units * K) return;
  const int u = (int)(gw / K);
  const int j = (int)(gw % K);
  const int idx = init_idx[(long)u * K + j];
  const bool valid = idx >= 0 && idx < m;
  const int row = valid ? n_sink + idx : 0;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(k_tok + ((size_t)u * capacity + row) * kHeadDim + 2 * lane);
  const double x0 = (double)bf16_lo(w), x1 = (double)bf16_hi(w);
  double n2 = x0 * x0 + x1 * x1;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) n2 += __shfl_xor(n2, o);
  uint32_t out = 0;
  if (valid && n2 > 0.0) {
    const double nrm = sqrt(n2);
    out = (uint32_t)f64_to_bf16_rne(x0 / nrm) | ((uint32_t)f64_to_bf16_rne(x1 / nrm) << 16);
  }
  *reinterpret_cast<uint32_t*>(cdir + ((size_t)u * K + j) * kHeadDim + 2 * lane) = out;
}

// Sum of squares, in f64 and in element order, of the 8 bf16 values of one
// 16-byte chunk of a key row: the per-chunk part of every key norm computed
// here.  A row's 16 chunk sums are then added by a butterfly over the chunk
// index (xor 1, 2, 4, 8), so wherever the norm is computed it is the same f64.
__device__ __forceinline__ double chunk_sq_sum(uint4 w) {
  double x[8];
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  double n2 = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) n2 += x[t] * x[t];
  return n2;
}

// ---------------------------------------------------------------------------
// Assignment: scores = X C^T on bf16 MFMA (v_mfma_f32_16x16x32_bf16), fp32
// accumulate, argmax fused in registers.  A workgroup owns 256 keys (4 waves x
// 4 tiles of 16 rows) held as MFMA A-operands in registers and walks the
// unit's directions in LDS chunks of 128.  Lane l of a 16x16 output tile holds
// column (direction) l%16 of rows 4*(l/16)..+3; the running best per row is
// kept per lane in increasing direction order (so ties keep the smaller
// index) and merged across the 16 lanes at the end.
// ---------------------------------------------------------------------------
constexpr int kAsMt = 4;                    // 16-row tiles per wave
constexpr int kAsRows = 4 * 16 * kAsMt;     // rows per workgroup
constexpr int kAsChunk = 128;               // directions per LDS chunk
constexpr int kAsLds = kHeadDim + 8;        // padded LDS row (272 B): conflict-free b128 reads

__global__ __launch_bounds__(256) void assign_kernel(const uint16_t* __restrict__ k_tok,
                                                     int capacity, int row0, int count,
                                                     const uint16_t* __restrict__ cdir, int K,
                                                     int32_t* __restrict__ assign, int clu_stride,
                                                     int first, int tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t cs[kAsChunk * kAsLds];
  const int u = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const int wrow0 = tile * kAsRows + wave * (16 * kAsMt);

  const uint16_t* kbase = k_tok + ((size_t)u * capacity + row0) * kHeadDim;
  bf16x8 a[kAsMt][4];
#pragma unroll
  for (int mt = 0; mt < kAsMt; ++mt) {
    int r = wrow0 + mt * 16 + r16;
    r = r < count ? r : count - 1;
    const uint16_t* src = kbase + (size_t)r * kHeadDim + kg * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s) a[mt][s] = *reinterpret_cast<const bf16x8*>(src + s * 32);
  }

  float best[kAsMt][4];
  int bidx[kAsMt][4];
#pragma unroll
  for (int mt = 0; mt < kAsMt; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      best[mt][i] = -INFINITY;
      bidx[mt][i] = 0;
    }

  const uint16_t* cbase = cdir + (size_t)u * K * kHeadDim;
  for (int c0 = 0; c0 < K; c0 += kAsChunk) {
    const int nc = min(kAsChunk, K - c0);
    const int ntile = (nc + 15) >> 4;
    __syncthreads();
    for (int e = threadIdx.x; e < ntile * 16 * 16; e += blockDim.x) {
      const int row = e >> 4, ch = e & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < nc) v = *reinterpret_cast<const uint4*>(cbase + (size_t)(c0 + row) * kHeadDim + ch * 8);
      *reinterpret_cast<uint4*>(cs + row * kAsLds + ch * 8) = v;
    }
    __syncthreads();
    // Full 16-direction tiles are software-pipelined: the MFMAs of tile t are
    // issued before the argmax of tile t-1, so the VALU epilogue overlaps them.
    const int nfull = nc >> 4;
    f32x4 acc[kAsMt], nxt[kAsMt];
    auto mfma_tile = [&](int t, f32x4* out) {
      bf16x8 b[4];
      const uint16_t* bp = cs + (t * 16 + r16) * kAsLds + kg * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) b[s] = *reinterpret_cast<const bf16x8*>(bp + s * 32);
#pragma unroll
      for (int mt = 0; mt < kAsMt; ++mt) out[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mt = 0; mt < kAsMt; ++mt)
          out[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][s], b[s], out[mt], 0, 0, 0);
    };
    auto argmax_tile = [&](const f32x4* in, int j) {
#pragma unroll
      for (int mt = 0; mt < kAsMt; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = in[mt][i];
          const bool gt = v > best[mt][i];
          best[mt][i] = gt ? v : best[mt][i];
          bidx[mt][i] = gt ? j : bidx[mt][i];
        }
    };
    if (nfull > 0) {
      mfma_tile(0, acc);
      for (int t = 1; t < nfull; ++t) {
        mfma_tile(t, nxt);
        argmax_tile(acc, c0 + (t - 1) * 16 + r16);
#pragma unroll
        for (int mt = 0; mt < kAsMt; ++mt) acc[mt] = nxt[mt];
      }
      argmax_tile(acc, c0 + (nfull - 1) * 16 + r16);
    }
    if (nc & 15) {  // last partial tile: columns past nc are padding
      mfma_tile(nfull, acc);
      if (nfull * 16 + r16 >= nc) {
#pragma unroll
        for (int mt = 0; mt < kAsMt; ++mt) acc[mt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
      argmax_tile(acc, c0 + nfull * 16 + r16);
    }
  }

#pragma unroll
  for (int mt = 0; mt < kAsMt; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float bv = best[mt][i];
      int bi = bidx[mt][i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      bidx[mt][i] = bi;
    }

  int32_t* out = assign + (size_t)u * clu_stride + first;
#pragma unroll
  for (int mt = 0; mt < kAsMt; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wrow0 + mt * 16 + kg * 4 + i;
      if (r16 == i && r < count) out[r] = bidx[mt][i];
    }
}

// ---------------------------------------------------------------------------
// Assignment with every direction resident in LDS (K <= 512): one workgroup of
// 12 waves per CU (three per SIMD) walks a range of 32-key tiles of one unit;
// each wave keeps the MFMA A-operands of its current tile in registers and
// loads the next tile's while the MFMAs of the current one run.  The
// directions are loaded into LDS once per workgroup instead of once per 256
// keys.  Two 16-key M-tiles per wave keep the kernel under 170 VGPRs, so a
// third wave per SIMD fits: the argmax VALU work of one wave then overlaps
// the MFMAs of two others (measured faster than three M-tiles at two waves
// per SIMD, whose B operands are reused more but hide less latency).
// ---------------------------------------------------------------------------
constexpr int kAsResWaves = 12;
constexpr int kAsResMt = 2;                  // 16-key M-tiles per wave tile (register budget)
constexpr int kAsResTile = 16 * kAsResMt;     // keys per wave tile
constexpr int kAsResMaxK = 512;

// NORMS: the kernel also writes 1/|x| (f64) of every key it assigns into
// invn[u, first + i], from the key registers it already holds (the chunk sums
// and butterfly of inv_norm_kernel, so the values are the same bits); the
// prefill's first round uses it instead of a separate pass over the keys.
// Labels go to assign (int32, row stride clu_stride) and / or assign16
// (uint16, row stride stride16), either of which may be null.
template <bool NORMS>
__global__ __launch_bounds__(kAsResWaves * 64) void assign_resident_kernel(
    const uint16_t* __restrict__ k_tok, int capacity, int row0, int count,
    const uint16_t* __restrict__ cdir, int K, int32_t* __restrict__ assign, int clu_stride, int first,
    int wg_per_unit, int tiles_per_wg, double* __restrict__ invn, uint16_t* __restrict__ assign16,
    int stride16) {
  extern __shared__ __attribute__((aligned(16))) uint16_t csr[];
  const int u = blockIdx.x / wg_per_unit;
  const int part = blockIdx.x % wg_per_unit;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int kg = lane >> 4;
  const int ntiles = (count + kAsResTile - 1) / kAsResTile;
  const int t0 = part * tiles_per_wg;
  const int t1 = min(ntiles, t0 + tiles_per_wg);
  if (t0 >= t1) return;  // uniform over the workgroup

  // all K directions (rows padded to a multiple of 16 with zeros)
  const int kpad = (K + 15) & ~15;
  const uint16_t* cbase = cdir + (size_t)u * K * kHeadDim;
  for (int e = threadIdx.x; e < kpad * 16; e += blockDim.x) {
    const int row = e >> 4, ch = e & 15;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < K) v = *reinterpret_cast<const uint4*>(cbase + (size_t)row * kHeadDim + ch * 8);
    *reinterpret_cast<uint4*>(csr + row * kAsLds + ch * 8) = v;
  }
  __syncthreads();

  const uint16_t* kbase = k_tok + ((size_t)u * capacity + row0) * kHeadDim;
  int32_t* out = assign != nullptr ? assign + (size_t)u * clu_stride + first : nullptr;
  uint16_t* out16 = assign16 != nullptr ? assign16 + (size_t)u * stride16 + first : nullptr;
  auto load_tile = [&](bf16x8 (&a)[kAsResMt][4], int t) {
#pragma unroll
    for (int mt = 0; mt < kAsResMt; ++mt) {
      int r = t * kAsResTile + mt * 16 + r16;
      r = r < count ? r : count - 1;
      const uint16_t* src = kbase + (size_t)r * kHeadDim + kg * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) a[mt][s] = *reinterpret_cast<const bf16x8*>(src + s * 32);
    }
  };
  auto compute_tile = [&](const bf16x8 (&a)[kAsResMt][4], int t) {
    // The MFMA takes the directions as its A operand and the keys as B, so
    // lane (r16 + 16 kg) gets directions 4 kg .. 4 kg + 3 of a block for key
    // r16 of each M-tile: the running best of a key over a block's 4 scores
    // is two max3 operations, and only the block index and its 4 scores are
    // kept when the best improves (strictly, so an earlier block wins ties).
    float best[kAsResMt];
    int bblk[kAsResMt];
    f32x4 bsc[kAsResMt];
#pragma unroll
    for (int mt = 0; mt < kAsResMt; ++mt) {
      best[mt] = -INFINITY;
      bblk[mt] = 0;
      bsc[mt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    // B operands (16 directions x 128 dims) of column block ct
    auto load_b = [&](bf16x8 (&b)[4], int ct) {
      const uint16_t* bp = csr + (ct * 16 + r16) * kAsLds + kg * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) b[s] = *reinterpret_cast<const bf16x8*>(bp + s * 32);
    };
    auto mfma_tile = [&](const bf16x8 (&b)[4], f32x4* o) {
#pragma unroll
      for (int mt = 0; mt < kAsResMt; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mt = 0; mt < kAsResMt; ++mt)
          o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[s], a[mt][s], o[mt], 0, 0, 0);
    };
    auto argmax_tile = [&](const f32x4* in, int blk) {
#pragma unroll
      for (int mt = 0; mt < kAsResMt; ++mt) {
        const float m3 = __builtin_fmaxf(__builtin_fmaxf(in[mt][0], in[mt][1]), in[mt][2]);
        const float m = __builtin_fmaxf(__builtin_fmaxf(m3, in[mt][3]), best[mt]);
        const bool gt = m > best[mt];
        bblk[mt] = gt ? blk : bblk[mt];
#pragma unroll
        for (int e = 0; e < 4; ++e) bsc[mt][e] = gt ? in[mt][e] : bsc[mt][e];
        best[mt] = m;
      }
    };
    // Two accumulator sets alternate; two B buffers alternate with blocks of
    // the same parity, each refilled right after its MFMAs issue, so an LDS
    // read has a whole block of MFMAs and argmax work to land in.
    const int nblk = (K + 15) >> 4;  // the last block may be partial (padded rows are zero)
    f32x4 acc0[kAsResMt], acc1[kAsResMt];
    bf16x8 b0[4], b1[4];
    load_b(b0, 0);
    if (nblk > 1) load_b(b1, 1);
    mfma_tile(b0, acc0);                        // block 0
    if (nblk > 2) load_b(b0, 2);
    int ct = 1;
    for (; ct + 3 < nblk; ct += 4) {            // four blocks per trip: fewer accumulator copies
      mfma_tile(b1, acc1);                      // block ct
      load_b(b1, ct + 2);
      argmax_tile(acc0, ct - 1);
      mfma_tile(b0, acc0);                      // block ct+1
      load_b(b0, ct + 3);
      argmax_tile(acc1, ct);
      mfma_tile(b1, acc1);                      // block ct+2
      if (ct + 4 < nblk) load_b(b1, ct + 4);
      argmax_tile(acc0, ct + 1);
      mfma_tile(b0, acc0);                      // block ct+3
      if (ct + 5 < nblk) load_b(b0, ct + 5);
      argmax_tile(acc1, ct + 2);
    }
    for (; ct + 1 < nblk; ct += 2) {
      mfma_tile(b1, acc1);                      // block ct (odd)
      if (ct + 2 < nblk) load_b(b1, ct + 2);
      argmax_tile(acc0, ct - 1);                // block ct-1
      mfma_tile(b0, acc0);                      // block ct+1 (even)
      if (ct + 3 < nblk) load_b(b0, ct + 3);
      argmax_tile(acc1, ct);                    // block ct
    }
    // acc0 holds block ct-1; block ct (odd, in b1), if any, is the last
    const bool tail = ct < nblk;
    if (tail) mfma_tile(b1, acc1);
    auto mask_pad = [&](f32x4* acc, int blk) {  // padded directions of a partial block never win
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (blk * 16 + 4 * kg + e >= K) {
#pragma unroll
          for (int mt = 0; mt < kAsResMt; ++mt) acc[mt][e] = -INFINITY;
        }
    };
    mask_pad(acc0, ct - 1);
    argmax_tile(acc0, ct - 1);
    if (tail) {
      mask_pad(acc1, ct);
      argmax_tile(acc1, ct);
    }
    // per key: the first of the kept block's 4 scores equal to the best, then
    // the best over the 4 lanes of the key (xor 16, 32); ties go to the
    // smaller index
#pragma unroll
    for (int mt = 0; mt < kAsResMt; ++mt) {
      float bv = best[mt];
      const f32x4 sc = bsc[mt];
      const int e = sc[0] == bv ? 0 : (sc[1] == bv ? 1 : (sc[2] == bv ? 2 : 3));
      int bi = bblk[mt] * 16 + 4 * kg + e;
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        const bool take = ov > bv || (ov == bv && oi < bi);
        bv = take ? ov : bv;
        bi = take ? oi : bi;
      }
      const int r = t * kAsResTile + mt * 16 + r16;
      if (kg == 0 && r < count) {
        if (out != nullptr) out[r] = bi;
        if (out16 != nullptr) out16[r] = (uint16_t)bi;
      }
    }
    if constexpr (NORMS) {
      // lane (r16, kg) holds chunks c = 4 s + kg of key r16: the butterfly's
      // xor 1 and 2 on c are lanes 16 and 32 apart, xor 4 and 8 are s ^ 1, s ^ 2
      double* inv_out = invn + (size_t)u * clu_stride + first;
#pragma unroll
      for (int mt = 0; mt < kAsResMt; ++mt) {
        double v[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v[s] = chunk_sq_sum(__builtin_bit_cast(uint4, a[mt][s]));
          v[s] += __shfl_xor(v[s], 16);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] += __shfl_xor(v[s], 32);
        const double n2 = (v[0] + v[1]) + (v[2] + v[3]);
        const int r = t * kAsResTile + mt * 16 + r16;
        if (kg == 0 && r < count) inv_out[r] = n2 > 0.0 ? 1.0 / sqrt(n2) : 0.0;
      }
    }
  };

  // tiles of this wave: t0 + wave, t0 + wave + 8, ...; two register sets alternate
  bf16x8 a0[kAsResMt][4], a1[kAsResMt][4];
  int t = t0 + wave;
  if (t < t1) load_tile(a0, t);
  for (; t < t1; t += 2 * kAsResWaves) {
    const int tn = t + kAsResWaves;
    if (tn < t1) load_tile(a1, tn);
    compute_tile(a0, t);
    if (tn >= t1) break;
    if (tn + kAsResWaves < t1) load_tile(a0, tn + kAsResWaves);
    compute_tile(a1, tn);
  }
}

// ---------------------------------------------------------------------------
// Lanes of the wave holding the same label as this lane (among `valid` lanes).
__device__ __forceinline__ unsigned long long match_label(int c, bool valid, int nbits) {
  unsigned long long peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (c >> b) & 1;
    const unsigned long long m = __ballot(valid && bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// ---------------------------------------------------------------------------
// Index build in one launch: the same stable counting sort by label (perm in
// cluster order, token order inside a cluster; offsets the exclusive scan of
// the cluster sizes), with the permutation written in whole lines.  A
// workgroup owns one (unit, range of clusters [c_lo, c_hi)); its 16 waves
// each own a contiguous segment of the unit's tokens.
//  1. Every wave walks its segment: a ballot counts its tokens below the
//     range, and LDS atomics count its in-range tokens per cluster (both
//     order-free).
//  2. The waves' below-counts give the range's first position; a scan over
//     the waves gives each wave's first position inside every cluster, and a
//     scan over the range's clusters their starts (written to offsets).
//  3. Every wave walks its segment again.  Per group of 8 batches of 64 it
//     compacts its in-range tokens, in token order, into an LDS list, then
//     places the list 64 at a time: rank among equal labels in lane order
//     plus the wave's running position of that cluster.  Token order inside
//     each cluster follows, as the sort is stable.
// Only in-range tokens reach the peer search, so the work per token that is
// repeated by every range's workgroup is a load, a ballot and a compare.
// The range's positions are staged in LDS and copied to perm contiguously; a
// range larger than the staging area writes its positions directly.
// ---------------------------------------------------------------------------
constexpr int kIdxThreads = 1024;
constexpr int kIdxWaves = kIdxThreads / kWave;
constexpr int kIdxPer = 32;                     // labels per lane loaded together
constexpr int kIdxFlush = 8;                    // batches compacted before placement
constexpr int kIdxBuf = kIdxFlush * kWave;      // compacted entries per wave
constexpr int kIdxLdsMax = 160 * 1024;          // LDS of one CU
constexpr int kIdxLabelBits = 10;               // range-relative label < kMaxClusters

static_assert(kMaxClusters <= (1 << kIdxLabelBits), "label field of a compacted entry");
static_assert(kMaxClusters <= kIdxThreads, "one thread per cluster of a range");

int index_ranges(int units, int K) {
  int p = (256 + units - 1) / units;  // about one workgroup per CU
  if (p > 32) p = 32;
  if (p > K) p = K;
  return p < 1 ? 1 : p;
}

int index_fixed_ints(int K, int ranges) {
  const int R = (K + ranges - 1) / ranges;
  return kIdxWaves * R + kIdxWaves * kIdxBuf + kIdxWaves + kIdxWaves + 1;
}

// staging room: twice a range's mean size, within what LDS leaves
int index_stage_ints(int K, int ranges, int count) {
  const int cap = kIdxLdsMax / (int)sizeof(int) - index_fixed_ints(K, ranges);
  const long per = ((long)count + ranges - 1) / ranges;
  long want = ((2 * per + 255) / 256) * 256;
  if (want < 1024) want = 1024;
  return (int)(want < cap ? want : cap);
}

__global__ __launch_bounds__(kIdxThreads) void index_kernel(const int32_t* __restrict__ assign, int clu_stride,
                                                            int count, int K, int ranges, int stage_cap,
                                                            int xcd_map, int n_sink,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ offsets) {
  extern __shared__ int ilds[];
  const int R = (K + ranges - 1) / ranges;
  int* cnt = ilds;                       // [waves][R] per-wave counts, then first positions
  int* buf = cnt + kIdxWaves * R;        // [waves][kIdxBuf] compacted (offset, label) entries
  int* below = buf + kIdxWaves * kIdxBuf;  // [waves] tokens below the range
  int* scr = below + kIdxWaves;          // [waves + 1] scan scratch
  int* stage = scr + kIdxWaves + 1;      // [stage_cap] the range's positions
  // Workgroups are dealt to the 8 XCDs round-robin; with xcd_map (units a
  // multiple of 8) all ranges of a unit share one XCD, so its labels are
  // fetched into that XCD's L2 once.
  const int b = blockIdx.x;
  const int u = xcd_map ? (b & 7) + 8 * ((b >> 3) / ranges) : b / ranges;
  const int p = xcd_map ? (b >> 3) % ranges : b % ranges;
  const int c_lo = (int)((long)K * p / ranges);
  const int c_hi = (int)((long)K * (p + 1) / ranges);
  const int nr = c_hi - c_lo;  // 1 <= nr <= R
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  for (int e = tid; e < kIdxWaves * R; e += kIdxThreads) cnt[e] = 0;
  __syncthreads();

  int rbits = 0;
  while ((1 << rbits) < nr) ++rbits;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t* a = assign + (size_t)u * clu_stride;
  const int seg = ((count + kIdxWaves - 1) / kIdxWaves + kWave - 1) & ~(kWave - 1);
  const int s_lo = min(count, wave * seg), s_hi = min(count, s_lo + seg);
  int* wc = cnt + wave * R;
  // A segment of one chunk keeps its labels in registers for both walks.
  const bool one_chunk = seg <= kIdxPer * kWave;  // uniform over the workgroup
  int cv[kIdxPer];
  auto load_chunk = [&](int b0) {
#pragma unroll
    for (int j = 0; j < kIdxPer; ++j) {
      const int i = b0 + j * kWave + lane;
      cv[j] = i < s_hi ? a[i] : 0;
    }
  };

  // 1. the segment's tokens below the range, and its in-range counts
  int nbelow = 0;
  for (int b0 = s_lo; b0 < s_hi; b0 += kIdxPer * kWave) {
    load_chunk(b0);
#pragma unroll
    for (int j = 0; j < kIdxPer; ++j) {
      if (b0 + j * kWave >= s_hi) break;  // uniform over the wave
      const bool valid = b0 + j * kWave + lane < s_hi;
      const int c = cv[j] < 0 ? 0 : (cv[j] >= K ? K - 1 : cv[j]);
      nbelow += __popcll(__ballot(valid && c < c_lo));
      if (valid && c >= c_lo && c < c_hi) atomicAdd(&wc[c - c_lo], 1);
    }
  }
  if (lane == 0) below[wave] = nbelow;
  __syncthreads();

  // 2. first positions, relative to the range's first position r_lo
  int r_lo = 0;
  for (int w = 0; w < kIdxWaves; ++w) r_lo += below[w];
  int size = 0;
  if (tid < nr) {
    for (int w = 0; w < kIdxWaves; ++w) {
      const int v = cnt[w * R + tid];
      cnt[w * R + tid] = size;
      size += v;
    }
  }
  int rtot;
  const int cs = block_exclusive_scan(size, scr, &rtot);  // size is 0 beyond the range
  if (tid < nr) {
    for (int w = 0; w < kIdxWaves; ++w) cnt[w * R + tid] += cs;
    offsets[(size_t)u * (K + 1) + c_lo + tid] = r_lo + cs;
  }
  if (p == ranges - 1 && tid == 0) offsets[(size_t)u * (K + 1) + K] = r_lo + rtot;
  __syncthreads();
  const bool staged = rtot <= stage_cap;  // uniform over the workgroup

  // 3. placement in token order
  int32_t* pu = perm + (size_t)u * clu_stride + r_lo;
  int* wb = buf + wave * kIdxBuf;
  for (int b0 = s_lo; b0 < s_hi; b0 += kIdxPer * kWave) {
    if (!one_chunk) load_chunk(b0);
#pragma unroll
    for (int g = 0; g < kIdxPer; g += kIdxFlush) {
      if (b0 + g * kWave >= s_hi) break;
      int nb = 0;  // compacted entries (uniform over the wave)
#pragma unroll
      for (int jj = 0; jj < kIdxFlush; ++jj) {
        const int j = g + jj;
        if (b0 + j * kWave >= s_hi) break;
        const int off = j * kWave + lane;
        const bool valid = b0 + off < s_hi;
        const int c = cv[j] < 0 ? 0 : (cv[j] >= K ? K - 1 : cv[j]);
        const bool mine = valid && c >= c_lo && c < c_hi;
        const unsigned long long m = __ballot(mine);
        if (mine) wb[nb + __popcll(m & lt)] = (off << kIdxLabelBits) | (c - c_lo);
        nb += __popcll(m);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int k0 = 0; k0 < nb; k0 += kWave) {
        const bool has = k0 + lane < nb;
        const int e = has ? wb[k0 + lane] : 0;
        const int cl = e & ((1 << kIdxLabelBits) - 1);
        const unsigned long long peers = match_label(cl, has, rbits);
        int pos = 0;
        if (has) pos = wc[cl] + __popcll(peers & lt);
        // every lane has read its base before the leader moves it
        if (has && (peers & lt) == 0ull) wc[cl] += __popcll(peers);
        if (has) {
          const int32_t tok = n_sink + b0 + (e >> kIdxLabelBits);
          if (staged)
            stage[pos] = tok;
          else
            pu[pos] = tok;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();  // the list is read before the next group overwrites it
    }
  }
  if (!staged) return;
  __syncthreads();
  for (int j = tid; j < rtot; j += kIdxThreads) pu[j] = stage[j];
}

// ---------------------------------------------------------------------------
// Lloyd rounds before the last: the sums move with the keys that changed
// cluster.  Round t's S_j = sum of x/|x| over the members of j is S_j of
// round t-1 plus the keys that joined j minus those that left; n_j likewise.
// S is held as exact integers, sum over members of rint(x_d / |x| * 2^F)
// (F = min(50, 62 - bitlen(m)), so no sum leaves int64), so the update by
// changes equals the sum from scratch bit for bit and does not depend on
// the order of the additions.  The rounding to 2^-F (at most 2^-48 per
// term at m < 2^15) is far below what f64 summation in any order already
// leaves.  Directions are then c_j = bf16(S_j / |S_j|) from S_j in f64, as
// in the update kernel.  The first round sums from scratch (index, then the
// update kernel's fixed mode) and the last rebuilds everything from the index;
// the rounds between move by the changes.
//
// A workgroup of 1024 threads owns one (unit, slice of D dims, range of
// clusters); with units >= 64 the range is all K clusters, so a key that
// changed cluster is read once per slice and leaves and joins in the same
// workgroup.  The range's additions sit in LDS as int64, one row of D + D/8
// slots per cluster (dim d of the slice at slot (D/8)(d % 8) + d / 8; the
// extra D/8 slots shift consecutive rows across the banks).  The 16 waves
// walk their token segments, compact the keys whose label changed (and whose
// old or new cluster is in the range), then add them D/8 lanes per key, 8
// dims (one 16-byte load) per lane, the next keys' loads in flight while the
// current ones are added.  A term is added as the bits of
// fma(x, 2^F/|x|, 1.5 * 2^52), whose integer value is the rounded term plus
// the bits of 1.5 * 2^52; the row's net member change times those bits is
// taken off at the end.  Each workgroup then adds its touched rows into S
// (slice 0 also moves n), and delta_dirs_kernel recomputes the directions
// from the whole rows.
// ---------------------------------------------------------------------------
constexpr int kDelThreads = 1024;
constexpr int kDelWaves = kDelThreads / kWave;
constexpr int kDelPer = 16;                   // label dwords (two tokens each) per lane loaded together
constexpr int kDelBuf = 8 * kWave;            // listed keys per wave
constexpr int kDelMaxRanges = 32;            // cluster ranges per unit


// dims per slice: the widest whose LDS rows for all K clusters fit beside the lists
int delta_dims(int K) { return K <= 440 ? 32 : 16; }

// bits of a range-relative label in a listed key (with one value for "none")
constexpr int delta_label_bits(int D) { return D == 32 ? 9 : 10; }

__host__ __device__ inline int delta_seg(int count) { return ((count + kDelWaves - 1) / kDelWaves + kWave - 1) & ~(kWave - 1); }



int delta_ranges(int units, int K) {
  const int slices = kHeadDim / delta_dims(K);
  int p = (256 + units * slices - 1) / (units * slices);  // about one workgroup per CU
  if (p > kDelMaxRanges) p = kDelMaxRanges;
  if (p > K) p = K;
  return p < 1 ? 1 : p;
}

size_t delta_lds_bytes(int K, int ranges) {
  const int D = delta_dims(K);
  const size_t R = (size_t)((K + ranges - 1) / ranges);
  return R * (D + D / 8) * sizeof(unsigned long long) + 2 * R * sizeof(int) +
         (size_t)kDelWaves * kDelBuf * sizeof(uint32_t);
}

// whether the delta rounds take this shape: the LDS rows fit and a wave's
// segment offsets fit their field of a listed key
bool delta_supported(int K, int count, int units) {
  // the rounds' 16-bit labels come from the resident assignment kernel
  if (K < 1 || K > kAsResMaxK || count < 1) return false;
  const int D = delta_dims(K);
  if (delta_lds_bytes(K, delta_ranges(units, K)) > (size_t)kIdxLdsMax) return false;
  return delta_seg(count) <= (1 << (32 - 2 * delta_label_bits(D)));
}

int delta_fbits(int m) {
  int b = 0;
  while (b < 31 && (1 << b) <= m) ++b;  // bitlen(m)
  const int f = 62 - b;
  return f < 50 ? f : 50;
}

template <int D>
__global__ __launch_bounds__(kDelThreads) void delta_kernel(
    const uint16_t* __restrict__ cur_lab, const uint16_t* __restrict__ prev_lab, int stride16, int clu_stride,
    int count, int K,
    int ranges, int xcd_map, const uint16_t* __restrict__ k_tok, int capacity, int n_sink,
    const double* __restrict__ invn, int fbits, long long* __restrict__ sfix, int32_t* __restrict__ csize) {
  constexpr int kSlices = kHeadDim / D;
  constexpr int LK = D / 8;       // lanes per key
  constexpr int KW = kWave / LK;  // keys per wave batch
  constexpr int ROW = D + LK;     // LDS slots per cluster row
  constexpr int kDelGroup = 2;   // key batches whose row loads are issued together
  // a listed key: token offset in the wave's segment, then the new and old
  // cluster relative to the range (kNone: outside it)
  constexpr int LB = delta_label_bits(D), OB = 32 - 2 * LB;
  constexpr uint32_t kNone = (1u << LB) - 1;
  extern __shared__ __align__(16) unsigned char dlds[];
  const int R = (K + ranges - 1) / ranges;
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(dlds);  // [R][ROW]
  int* dn = reinterpret_cast<int*>(acc + (size_t)R * ROW);                // [R] member count changes
  int* touched = dn + R;                                                   // [R]
  uint32_t* buf = reinterpret_cast<uint32_t*>(touched + R);                // [waves][kDelBuf] listed keys
  // Workgroups are dealt to the 8 XCDs round-robin; with xcd_map (units a
  // multiple of 8) all workgroups of a unit share one XCD.
  const int P = kSlices * ranges;
  const int b = blockIdx.x;
  const int u = xcd_map ? (b & 7) + 8 * ((b >> 3) / P) : b / P;
  const int q = xcd_map ? (b >> 3) % P : b % P;
  const int slice = q % kSlices, p = q / kSlices;
  const int c_lo = (int)((long)K * p / ranges);
  const int c_hi = (int)((long)K * (p + 1) / ranges);
  const int nr = c_hi - c_lo;  // 1 <= nr <= R
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  for (int e = tid; e < nr * ROW; e += kDelThreads) acc[e] = 0ull;
  for (int e = tid; e < nr; e += kDelThreads) dn[e] = touched[e] = 0;
  __syncthreads();

  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // a unit's labels as dwords of two (stride16 and the segments' starts are even)
  const uint32_t* cu = reinterpret_cast<const uint32_t*>(cur_lab + (size_t)u * stride16);
  const uint32_t* pu = reinterpret_cast<const uint32_t*>(prev_lab + (size_t)u * stride16);
  const int seg = delta_seg(count);
  const int s_lo = min(count, wave * seg), s_hi = min(count, s_lo + seg);
  uint32_t* wb = buf + wave * kDelBuf;
  const int kk = lane / LK, lk = lane % LK;
  const uint16_t* ku = k_tok + ((size_t)u * capacity + n_sink) * kHeadDim + slice * D + 8 * lk;
  const double* iu = invn + (size_t)u * clu_stride;
  const double scale = __builtin_ldexp(1.0, fbits);
  const double magic = 6755399441055744.0;  // 1.5 * 2^52: adding it rounds to an integer
  const long long magic_bits = __double_as_longlong(magic);

  // KW keys per batch, kDelGroup batches per load group, two groups in flight
  auto load_group = [&](int k0, int nb, uint4(&x)[kDelGroup], double(&iv)[kDelGroup],
                        uint32_t(&ent)[kDelGroup]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kDelGroup; ++s) {
      const int k = k0 + s * KW + kk;
      ent[s] = k < nb ? wb[k] : 0xffffffffu;
      if (k < nb) {
        const int i = s_lo + (int)(ent[s] & ((1u << OB) - 1));
        x[s] = *reinterpret_cast<const uint4*>(ku + (size_t)i * kHeadDim);
        iv[s] = iu[i];
      }
    }
  };
  auto add_group = [&](const uint4(&x)[kDelGroup], const double(&iv)[kDelGroup],
                       const uint32_t(&ent)[kDelGroup]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < kDelGroup; ++s) {
      if (ent[s] == 0xffffffffu) continue;
      const uint32_t cr = (ent[s] >> OB) & kNone, pr = ent[s] >> (OB + LB);
      const uint32_t w[4] = {x[s].x, x[s].y, x[s].z, x[s].w};
      const double ivf = iv[s] * scale;
      unsigned long long* rc = acc + (size_t)cr * ROW + lk;
      unsigned long long* rp = acc + (size_t)pr * ROW + lk;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
        const unsigned long long v =
            (unsigned long long)__double_as_longlong(fma((double)__uint_as_float(h), ivf, magic));
        if (cr != kNone) atomicAdd(rc + LK * e, v);
        if (pr != kNone) atomicSub(rp + LK * e, v);
      }
    }
  };
  // add the wave's listed keys, then empty the list
  auto drain = [&](int nb) __attribute__((always_inline)) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    constexpr int kStep = kDelGroup * KW;
    uint4 xa[kDelGroup], xb[kDelGroup];
    double ia[kDelGroup], ib[kDelGroup];
    uint32_t ea[kDelGroup], eb[kDelGroup];
    if (nb > 0) load_group(0, nb, xa, ia, ea);
    for (int k0 = 0; k0 < nb; k0 += 2 * kStep) {
      if (k0 + kStep < nb) load_group(k0 + kStep, nb, xb, ib, eb);
      add_group(xa, ia, ea);
      if (k0 + kStep >= nb) break;
      if (k0 + 2 * kStep < nb) load_group(k0 + 2 * kStep, nb, xa, ia, ea);
      add_group(xb, ib, eb);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the list is read before it is refilled
  };

  // Each wave walks its token segment in chunks of 2 kDelPer batches, with
  // both rounds' labels of a chunk loaded together as dwords of two tokens
  // (one load round trip per chunk: a whole segment at the benchmark's
  // shapes).  It lists the keys that changed cluster whose new or old cluster
  // is in the range, and adds them when the list could not take 4 more
  // batches, so a round with few changes pays few row loads.
  int nb = 0;  // listed keys (uniform over the wave)
  for (int b0 = s_lo; b0 < s_hi; b0 += 2 * kDelPer * kWave) {
    uint32_t cd[kDelPer], od[kDelPer];
#pragma unroll
    for (int j = 0; j < kDelPer; ++j) {
      const int i = b0 + 2 * (j * kWave + lane);  // even: tokens i and i + 1
      cd[j] = i < s_hi ? cu[i >> 1] : 0u;
      od[j] = i < s_hi ? pu[i >> 1] : 0u;
    }
    // one token per lane of dword j (h = 0: its low label, 1: its high one)
    auto list_batch = [&](int j, int h, uint32_t cdw, uint32_t odw) __attribute__((always_inline)) {
      const int i = b0 + 2 * (j * kWave + lane) + h;
      const int c_raw = (int)(h ? cdw >> 16 : cdw & 0xffffu), o_raw = (int)(h ? odw >> 16 : odw & 0xffffu);
      const int c = c_raw >= K ? K - 1 : c_raw;
      const int o = o_raw >= K ? K - 1 : o_raw;
      const bool moved = c != o;
      const bool cin = i < s_hi && moved && c >= c_lo && c < c_hi;
      const bool pin = i < s_hi && moved && o >= c_lo && o < c_hi;
      if (cin) {
        atomicAdd(&dn[c - c_lo], 1);
        touched[c - c_lo] = 1;
      }
      if (pin) {
        atomicAdd(&dn[o - c_lo], -1);
        touched[o - c_lo] = 1;
      }
      const bool mine = cin || pin;
      const unsigned long long m = __ballot(mine);
      if (mine)
        wb[nb + __popcll(m & lt)] = (uint32_t)(i - s_lo) | ((cin ? (uint32_t)(c - c_lo) : kNone) << OB) |
                                    ((pin ? (uint32_t)(o - c_lo) : kNone) << (OB + LB));
      nb += __popcll(m);
    };
    // two dwords (four batches) at a time, the list drained first when it
    // could not take them
#pragma unroll
    for (int j0 = 0; j0 < kDelPer; j0 += 2) {
      if (b0 + 2 * j0 * kWave >= s_hi) break;  // uniform over the wave
      if (nb > kDelBuf - 4 * kWave) {
        drain(nb);
        nb = 0;
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        list_batch(j0 + jj, 0, cd[j0 + jj], od[j0 + jj]);
        list_batch(j0 + jj, 1, cd[j0 + jj], od[j0 + jj]);
      }
    }
  }
  drain(nb);
  __syncthreads();

  // This slice of the touched rows into S (LK lanes per row, 8 dims each);
  // slice 0 also moves n.
  for (int r = wave * KW + kk; r < nr; r += kDelWaves * KW) {
    if (touched[r] == 0) continue;
    const size_t j = (size_t)u * K + c_lo + r;
    const size_t sidx = j * kHeadDim + slice * D + 8 * lk;
    // net members added times the bits of 1.5 * 2^52 come off every slot
    const unsigned long long bias = (unsigned long long)(long long)dn[r] * (unsigned long long)magic_bits;
    long long sf[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const long long add = (long long)(acc[(size_t)r * ROW + LK * t + lk] - bias);
      sf[t] = sfix[sidx + t] + add;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) sfix[sidx + t] = sf[t];
    if (slice == 0 && lk == 0) csize[j] += dn[r];
  }
}


// c_j = bf16(S_j / |S_j|) from the fixed-point sums where n_j > 0 and
// S_j != 0 (otherwise c_j stays): 16 lanes per cluster row, 8 dims each.
__global__ __launch_bounds__(1024) void delta_dirs_kernel(const long long* __restrict__ sfix,
                                                          const int32_t* __restrict__ csize,
                                                          uint16_t* __restrict__ cdir, long rows, int fbits) {
  const long row = (long)blockIdx.x * 64 + (threadIdx.x >> 4);
  if (row >= rows) return;  // whole 16-lane groups leave together
  const int li = threadIdx.x & 15;
  const size_t sidx = (size_t)row * kHeadDim + li * 8;
  const double unscale = __builtin_ldexp(1.0, -fbits);
  double sv[8];
  double ns2 = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    sv[t] = (double)sfix[sidx + t] * unscale;
    ns2 += sv[t] * sv[t];
  }
  ns2 = xor_sum16(ns2);
  if (csize[row] > 0 && ns2 > 0.0) {
    const double nrm = sqrt(ns2);
    uint32_t wv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      wv[t] = (uint32_t)f64_to_bf16_rne(sv[2 * t] / nrm) | ((uint32_t)f64_to_bf16_rne(sv[2 * t + 1] / nrm) << 16);
    *reinterpret_cast<uint4*>(cdir + sidx) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// ---------------------------------------------------------------------------
// Inverse key norms 1/|x| (f64) of clustered tokens [first, first + count):
// 16 lanes per row, kNormRows rows per 16-lane group with all their loads in
// flight (a workgroup covers 16 * kNormRows consecutive rows, each load
// instruction of it 16 consecutive rows).  Computed once per prefill /
// incremental call; the update kernels reuse them every Lloyd round.
// ---------------------------------------------------------------------------
constexpr int kNormRows = 4;

__global__ __launch_bounds__(256) void inv_norm_kernel(const uint16_t* __restrict__ k_tok, int capacity,
                                                       int n_sink, int first, int count,
                                                       double* __restrict__ invn, int clu_stride,
                                                       int rows_per_unit_blocks) {
  const int u = blockIdx.x / rows_per_unit_blocks;
  const int b = blockIdx.x % rows_per_unit_blocks;
  const int li = threadIdx.x & 15;
  const int i0 = b * (16 * kNormRows) + (threadIdx.x >> 4);
  const uint16_t* ku = k_tok + ((size_t)u * capacity + n_sink + first) * kHeadDim + li * 8;
  uint4 w[kNormRows];
#pragma unroll
  for (int k = 0; k < kNormRows; ++k) {
    const int i = i0 + 16 * k;
    w[k] = *reinterpret_cast<const uint4*>(ku + (size_t)(i < count ? i : 0) * kHeadDim);
  }
#pragma unroll
  for (int k = 0; k < kNormRows; ++k) {
    const int i = i0 + 16 * k;
    const double n2 = xor_sum16(chunk_sq_sum(w[k]));
    if (i < count && li == 0) invn[(size_t)u * clu_stride + first + i] = n2 > 0.0 ? 1.0 / sqrt(n2) : 0.0;
  }
}

// ---------------------------------------------------------------------------
// Update: one wave per (unit, cluster); 16 member rows per step, one row per
// 16-lane group at a time (8 dims per lane), all 4 row loads of a group issued
// together.  Sums in f64: S_j = sum x/|x| (with the precomputed 1/|x|),
// M_j = sum x.  Iteration mode rebuilds S from scratch and refreshes the
// direction; final mode also writes M, the mean and the cluster-ordered K/V
// rows; incremental mode adds only the members past the old size (new tokens
// sort last in their cluster), keeps the old sums, refreshes touched clusters
// and rewrites every row.
// ---------------------------------------------------------------------------
// OWN_NORMS: 1/|x| of each row is computed from the row itself (the 16 lanes
// that hold it, in the same order as inv_norm_kernel, so the value is the
// same) instead of being read from invn; for a single pass over the keys this
// saves the separate norm pass.
//
// Fixed mode (a Lloyd round followed by rounds by changes): as the iteration
// mode, but S is summed as the exact fixed-point integers of the rounds by
// changes (rint(x_d / |x| * 2^fbits) as int64, written over csum) and the
// direction is computed from them as delta_dirs_kernel does.
template <int MODE, bool OWN_NORMS>
__global__ __launch_bounds__(256) void update_kernel(
    const uint16_t* __restrict__ k_tok, const uint16_t* __restrict__ v_tok, int capacity, int n_sink,
    const int32_t* __restrict__ perm, int clu_stride, const int32_t* __restrict__ offsets, int K,
    const double* __restrict__ invn, double* __restrict__ csum, double* __restrict__ msum,
    float* __restrict__ cmean, int32_t* __restrict__ csize, uint16_t* __restrict__ cdir,
    uint16_t* __restrict__ k_dst, uint16_t* __restrict__ v_dst, int units, int fbits) {
  constexpr bool FX = MODE == kUpdFixed;
  constexpr bool ITER = MODE == kUpdIter || FX;  // sums and directions only
  const int lane = lane_id();
  const long gw = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= (long)units * K) return;
  const int u = (int)(gw / K);
  const int j = (int)(gw % K);
  const int g = lane >> 4;
  const int li = lane & 15;
  const int lo = offsets[(size_t)u * (K + 1) + j];
  const int hi = offsets[(size_t)u * (K + 1) + j + 1];
  const int n = hi - lo;
  const size_t sidx = ((size_t)u * K + j) * kHeadDim + li * 8;
  const int n_old = (MODE == kUpdIncr) ? csize[(size_t)u * K + j] : 0;
  const int acc_from = lo + n_old;

  double s[8], mm[8];
  long long sf[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    s[t] = mm[t] = 0.0;
    sf[t] = 0ll;
  }
  const double fx_scale = __builtin_ldexp(1.0, fbits);
  const double fx_magic = 6755399441055744.0;  // 1.5 * 2^52, as in the rounds by changes
  const long long fx_magic_bits = __double_as_longlong(fx_magic);

  const int32_t* pu = perm + (size_t)u * clu_stride;
  const double* iu = OWN_NORMS ? nullptr : invn + (size_t)u * clu_stride;
  const uint16_t* ku = k_tok + (size_t)u * capacity * kHeadDim + li * 8;
  const uint16_t* vu = v_tok + (size_t)u * capacity * kHeadDim + li * 8;
  for (int p0 = lo; p0 < hi; p0 += 16) {
    int tk = 0;
    double iv = 0.0;
    const int pl = p0 + lane;
    if (lane < 16 && pl < hi) {
      tk = pu[pl];
      tk = tk < n_sink ? n_sink : (tk >= capacity ? capacity - 1 : tk);
      if (!OWN_NORMS && pl >= acc_from) iv = iu[tk - n_sink];
    }
    int tks[4];
    double ivs[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tks[k] = __shfl(tk, 4 * k + g);
      ivs[k] = __shfl(iv, 4 * k + g);
    }
    uint4 kx[4], vx[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = p0 + 4 * k + g;
      if (p < hi) {
        kx[k] = *reinterpret_cast<const uint4*>(ku + (size_t)tks[k] * kHeadDim);
        if (!ITER) vx[k] = *reinterpret_cast<const uint4*>(vu + (size_t)tks[k] * kHeadDim);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = p0 + 4 * k + g;
      if (p >= hi) continue;
      if (!ITER) {
        *reinterpret_cast<uint4*>(k_dst + ((size_t)u * clu_stride + p) * kHeadDim + li * 8) = kx[k];
        *reinterpret_cast<uint4*>(v_dst + ((size_t)u * clu_stride + p) * kHeadDim + li * 8) = vx[k];
      }
      if (p < acc_from) continue;
      double x[8];
      x[0] = bf16_lo(kx[k].x); x[1] = bf16_hi(kx[k].x);
      x[2] = bf16_lo(kx[k].y); x[3] = bf16_hi(kx[k].y);
      x[4] = bf16_lo(kx[k].z); x[5] = bf16_hi(kx[k].z);
      x[6] = bf16_lo(kx[k].w); x[7] = bf16_hi(kx[k].w);
      double ivk = ivs[k];
      if (OWN_NORMS) {
        double n2 = 0.0;
#pragma unroll
        for (int t = 0; t < 8; ++t) n2 += x[t] * x[t];
        n2 = xor_sum16(n2);
        ivk = n2 > 0.0 ? 1.0 / sqrt(n2) : 0.0;
      }
      if constexpr (FX) {
        const double ivf = ivk * fx_scale;
#pragma unroll
        for (int t = 0; t < 8; ++t) sf[t] += __double_as_longlong(fma(x[t], ivf, fx_magic)) - fx_magic_bits;
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          s[t] = fma(x[t], ivk, s[t]);
          if (!ITER) mm[t] += x[t];
        }
      }
    }
  }
  if constexpr (FX) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      sf[t] += __shfl_xor(sf[t], 16);
      sf[t] += __shfl_xor(sf[t], 32);
      s[t] = (double)sf[t] * __builtin_ldexp(1.0, -fbits);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      s[t] += __shfl_xor(s[t], 16);
      s[t] += __shfl_xor(s[t], 32);
      if (!ITER) {
        mm[t] += __shfl_xor(mm[t], 16);
        mm[t] += __shfl_xor(mm[t], 32);
      }
    }
  }
  if (MODE == kUpdIncr) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      s[t] += csum[sidx + t];
      mm[t] += msum[sidx + t];
    }
  }
  double ns2 = 0.0;
#pragma unroll
  for (int t = 0; t < 8; ++t) ns2 += s[t] * s[t];
  ns2 = xor_sum16(ns2);
  if (g != 0) return;

  if constexpr (FX) {
#pragma unroll
    for (int t = 0; t < 8; ++t) reinterpret_cast<long long*>(csum)[sidx + t] = sf[t];
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) csum[sidx + t] = s[t];
  }
  const bool touched = (MODE == kUpdIncr) ? (n > n_old) : (n > 0);
  if (touched && ns2 > 0.0) {
    const double nrm = sqrt(ns2);
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w[t] = (uint32_t)f64_to_bf16_rne(s[2 * t] / nrm) | ((uint32_t)f64_to_bf16_rne(s[2 * t + 1] / nrm) << 16);
    *reinterpret_cast<uint4*>(cdir + sidx) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (!ITER) {
    float mu[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      msum[sidx + t] = mm[t];
      mu[t] = n > 0 ? (float)(mm[t] / (double)n) : 0.0f;
    }
    *reinterpret_cast<float4*>(cmean + sidx) = make_float4(mu[0], mu[1], mu[2], mu[3]);
    *reinterpret_cast<float4*>(cmean + sidx + 4) = make_float4(mu[4], mu[5], mu[6], mu[7]);
  }
  if (li == 0) csize[(size_t)u * K + j] = n;
}

// ---------------------------------------------------------------------------
// Drift split.  The drift of cluster j is 1 - |S_j| / n_j (f64 unit-key sums).
// Clusters with n_j >= 2 and drift above the threshold are ranked by drift
// (descending, ties to the smaller index) and paired with the empty slots in
// index order.  For a pair (j, f) the member with the smallest cosine to c~_j
// (ties to the earliest position, which is the earliest token inside a
// cluster) seeds f with bf16(x / |x|); then every member of j takes the larger
// of x . c~_j and x . c~_f (ties to the smaller slot).  Every dot product is
// f64 over bf16 values: the products are exact, so these decisions do not
// depend on the summation order.  Only the labels are written here; the caller
// rebuilds the index, sums, directions, means and cluster-ordered rows.
//
// split_plan_kernel (one workgroup per unit) writes the pairs to a plan
// [units, 2K + 1] int32: the pair count, then j of each pair, then f.
// split_move_kernel spreads a unit's pairs over kSplitPar workgroups.  Pairs
// touch disjoint members, so the workgroups write disjoint labels.  A member
// row is read from the cluster-ordered copy (a cluster's rows are contiguous
// there) as one 16-byte load per lane (16 lanes per row, 8 dims each); a wave
// holds 16 rows in flight and a workgroup 64.  A cluster of at most 64 rows is
// read once: its rows stay in registers from the seed search to the move.
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 4;
constexpr int kSplitMaxK = 1024;  // the layer's cluster limit; per-unit lists live in LDS
constexpr int kSplitPar = 16;     // workgroups per unit in the move kernel
constexpr int kSplitPlanUnroll = 8;
constexpr int kSplitMoveWaves = 4;
constexpr int kSplitSlotRows = 4;                              // rows per 16-lane slot in flight
constexpr int kSplitRows = kSplitMoveWaves * 4 * kSplitSlotRows;  // rows per workgroup step

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(kSplitWaves * 64) void split_plan_kernel(
    int K, const double* __restrict__ csum, const int32_t* __restrict__ csize, double threshold,
    int32_t* __restrict__ plan) {
  constexpr int kPer = kSplitMaxK / (kSplitWaves * 64);  // clusters per thread for sizes and free slots
  __shared__ double s_drift[kSplitMaxK];   // drift of a candidate, -inf otherwise
  __shared__ int s_free[kSplitMaxK];       // empty slots, ascending
  __shared__ int s_scan[kSplitWaves + 1];
  __shared__ int s_bp[kSplitWaves];

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid >> 6;
  const int32_t* nu = csize + (size_t)u * K;
  int32_t* pl = plan + (size_t)u * (2 * K + 1);

  // sizes of clusters kPer t .. kPer t + kPer - 1 (all loads in flight), and
  // this thread's empty ones
  int n_own[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = kPer * tid + i;
    n_own[i] = j < K ? nu[j] : -1;
  }
  // |S_j|^2 into s_drift: 16 lanes per cluster (8 f64 each), 4 clusters per
  // wave, and kSplitPlanUnroll of them per lane slot in flight at once
  {
    const int grp = lane >> 4, sub = lane & 15;
    for (int j0 = wv * 4 + grp; j0 < K; j0 += kSplitWaves * 4 * kSplitPlanUnroll) {
      double2 sv[kSplitPlanUnroll][4];
#pragma unroll
      for (int t = 0; t < kSplitPlanUnroll; ++t) {
        const int j = min(j0 + t * kSplitWaves * 4, K - 1);
        const double2* row = reinterpret_cast<const double2*>(csum + ((size_t)u * K + j) * kHeadDim + 8 * sub);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[t][i] = row[i];
      }
#pragma unroll
      for (int t = 0; t < kSplitPlanUnroll; ++t) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = fma(sv[t][i].x, sv[t][i].x, fma(sv[t][i].y, sv[t][i].y, ss));
        ss = xor_sum16(ss);
        const int j = j0 + t * kSplitWaves * 4;
        if (sub == 0 && j < K) s_drift[j] = ss;
      }
    }
  }
  int my_free = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) my_free += n_own[i] == 0 ? 1 : 0;
  int nfree = 0;
  // (its barriers also order the |S_j|^2 writes above before the reads below)
  const int fo = block_exclusive_scan(my_free, s_scan, &nfree);
#pragma unroll
  for (int i = 0, f = fo; i < kPer; ++i)
    if (n_own[i] == 0) s_free[f++] = kPer * tid + i;
  // drift 1 - |S_j| / n_j of this thread's clusters; -inf unless a candidate
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = kPer * tid + i;
    if (j < K) {
      const int n = n_own[i];
      const double d = n > 0 ? 1.0 - sqrt(s_drift[j]) / (double)n : 0.0;
      s_drift[j] = (n >= 2 && d > threshold) ? d : -INFINITY;
    }
  }
  __syncthreads();
  int my_cand = 0;
  for (int j = tid; j < K; j += kSplitWaves * 64) {
    const double dj = s_drift[j];
    if (dj == -INFINITY) continue;
    ++my_cand;
    int r = 0;
    for (int i = 0; i < K; ++i) {
      const double di = s_drift[i];
      r += (di > dj || (di == dj && i < j)) ? 1 : 0;
    }
    if (r < nfree) {
      pl[1 + r] = j;
      pl[1 + K + r] = s_free[r];
    }
  }
  for (int o = 1; o < kWave; o <<= 1) my_cand += __shfl_xor(my_cand, o);
  if (lane == 0) s_bp[wv] = my_cand;
  __syncthreads();
  if (tid == 0) {
    int pairs = 0;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) pairs += s_bp[w];
    pl[0] = pairs < nfree ? pairs : nfree;
  }
}

// 8 dims of one bf16 row as f64 (exact).
__device__ __forceinline__ void widen8(const uint4 w, double* x) {
  x[0] = (double)bf16_lo(w.x); x[1] = (double)bf16_hi(w.x);
  x[2] = (double)bf16_lo(w.y); x[3] = (double)bf16_hi(w.y);
  x[4] = (double)bf16_lo(w.z); x[5] = (double)bf16_hi(w.z);
  x[6] = (double)bf16_lo(w.w); x[7] = (double)bf16_hi(w.w);
}

__device__ __forceinline__ double dot8(const double* a, const double* b) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fma(a[i], b[i], s);
  return s;
}

__global__ __launch_bounds__(kSplitMoveWaves * 64) void split_move_kernel(
    const uint16_t* __restrict__ k_clu, int n_sink, const int32_t* __restrict__ perm, int clu_stride,
    const int32_t* __restrict__ offsets, int K, const uint16_t* __restrict__ cdir,
    const int32_t* __restrict__ plan, int32_t* __restrict__ assign) {
  __shared__ double s_bc[kSplitMoveWaves * 4];
  __shared__ int s_bp[kSplitMoveWaves * 4];

  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid >> 6;
  const int grp = lane >> 4;   // row slot of the wave
  const int sub = lane & 15;   // 8-dim slice of the row
  const int32_t* pl = plan + (size_t)u * (2 * K + 1);
  const int pairs = pl[0];
  const int32_t* pu = perm + (size_t)u * clu_stride;
  // the cluster-ordered copy: position p holds the key of token perm[p]
  const uint16_t* ku = k_clu + (size_t)u * clu_stride * kHeadDim + 8 * sub;
  int32_t* au = assign + (size_t)u * clu_stride;
  const int slot0 = wv * 4 * kSplitSlotRows + grp;

  for (int r = blockIdx.y; r < pairs; r += gridDim.y) {
    const int j = pl[1 + r];
    const int f = pl[1 + K + r];
    const int lo = min(max(offsets[(size_t)u * (K + 1) + j], 0), clu_stride);
    const int hi = min(max(offsets[(size_t)u * (K + 1) + j + 1], lo), clu_stride);
    const bool one_step = hi - lo <= kSplitRows;  // rows stay in registers for the move
    double cj[8];
    widen8(*reinterpret_cast<const uint4*>(cdir + ((size_t)u * K + j) * kHeadDim + 8 * sub), cj);

    // seed: the member with the smallest cosine to c~_j, earliest position on ties
    double best = INFINITY;
    int bestp = 0x7fffffff;
    uint4 w[kSplitSlotRows];
    for (int base = lo + slot0; base < hi; base += kSplitRows) {
#pragma unroll
      for (int t = 0; t < kSplitSlotRows; ++t) {
        const int p = min(base + 4 * t, hi - 1);
        w[t] = *reinterpret_cast<const uint4*>(ku + (size_t)p * kHeadDim);
      }
#pragma unroll
      for (int t = 0; t < kSplitSlotRows; ++t) {
        double x[8];
        widen8(w[t], x);
        const double dot = xor_sum16(dot8(x, cj));
        const double ss = xor_sum16(dot8(x, x));
        const double cs = ss > 0.0 ? dot / sqrt(ss) : 0.0;
        if (base + 4 * t < hi && cs < best) {  // a slot's positions ascend: the first minimum stays
          best = cs;
          bestp = base + 4 * t;
        }
      }
    }
    if (sub == 0) {
      s_bc[wv * 4 + grp] = best;
      s_bp[wv * 4 + grp] = bestp;
    }
    __syncthreads();
    int sp = s_bp[0];
    double sb = s_bc[0];
#pragma unroll
    for (int g = 1; g < kSplitMoveWaves * 4; ++g) {
      if (s_bc[g] < sb || (s_bc[g] == sb && s_bp[g] < sp)) {
        sb = s_bc[g];
        sp = s_bp[g];
      }
    }
    __syncthreads();  // s_bc / s_bp are rewritten by the next pair
    if (sp < lo || sp >= hi) continue;  // no members (cannot happen for n_j >= 2); uniform
    double sx[8];
    widen8(*reinterpret_cast<const uint4*>(ku + (size_t)sp * kHeadDim), sx);
    const double sss = xor_sum16(dot8(sx, sx));
    double cf[8];
    const double nrm = sqrt(sss);
#pragma unroll
    for (int i = 0; i < 8; ++i) cf[i] = sss > 0.0 ? (double)bf16_to_f32(f64_to_bf16_rne(sx[i] / nrm)) : 0.0;

    // move: each member of j takes the larger score of c~_j and c~_f
    for (int base = lo + slot0; base < hi; base += kSplitRows) {
      int tk[kSplitSlotRows];
#pragma unroll
      for (int t = 0; t < kSplitSlotRows; ++t) {
        const int p = min(base + 4 * t, hi - 1);
        tk[t] = pu[p];
        if (!one_step) w[t] = *reinterpret_cast<const uint4*>(ku + (size_t)p * kHeadDim);
      }
#pragma unroll
      for (int t = 0; t < kSplitSlotRows; ++t) {
        double x[8];
        widen8(w[t], x);
        const double sj = xor_sum16(dot8(x, cj));
        const double sf = xor_sum16(dot8(x, cf));
        const bool move = f < j ? (sf >= sj) : (sf > sj);
        const int row = tk[t] - n_sink;
        if (base + 4 * t < hi && move && sub == 0 && row >= 0 && row < clu_stride) au[row] = f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_init_dirs(const uint16_t* k_tok, int capacity, int n_sink, int m,
                            const int32_t* init_idx, int K, uint16_t* cdir, int units,
                            hipStream_t s) {
  const long waves = (long)units * K;
  hipLaunchKernelGGL(init_dirs_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, k_tok,
                     capacity, n_sink, m, init_idx, K, cdir, units);
  return hipGetLastError();
}

hipError_t launch_assign(const uint16_t* k_tok, int capacity, int row0, int count,
                         const uint16_t* cdir, int K, int32_t* assign, int clu_stride,
                         int first, int units, hipStream_t s, double* invn, uint16_t* assign16,
                         int stride16) {
  if (count <= 0) return hipSuccess;
  if (assign16 != nullptr && K > kAsResMaxK) return hipErrorInvalidValue;  // the resident kernel only
  if (K <= kAsResMaxK) {
    // about one 8-wave workgroup per CU, each on one unit's range of key tiles
    const int ntiles = (count + kAsResTile - 1) / kAsResTile;
    int wpu = (256 + units - 1) / units;
    const int max_wpu = (ntiles + kAsResWaves - 1) / kAsResWaves;
    if (wpu > max_wpu) wpu = max_wpu;
    if (wpu < 1) wpu = 1;
    const int tpw = (ntiles + wpu - 1) / wpu;
    const size_t lds = (size_t)((K + 15) & ~15) * kAsLds * sizeof(uint16_t);
    // dynamic LDS above 64 KiB must be allowed explicitly; set once per
    // process (calls may come from several host threads)
    static std::once_flag lds_once;
    static hipError_t lds_status = hipSuccess;
    std::call_once(lds_once, [] {
      const int bytes = (int)(kAsResMaxK * kAsLds * sizeof(uint16_t));
      lds_status = hipFuncSetAttribute((const void*)assign_resident_kernel<false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (lds_status == hipSuccess)
        lds_status = hipFuncSetAttribute((const void*)assign_resident_kernel<true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    });
    if (lds_status != hipSuccess) return lds_status;
    if (invn != nullptr)
      hipLaunchKernelGGL(assign_resident_kernel<true>, dim3((unsigned)(units * wpu)), dim3(kAsResWaves * 64), lds,
                         s, k_tok, capacity, row0, count, cdir, K, assign, clu_stride, first, wpu, tpw, invn,
                         assign16, stride16);
    else
      hipLaunchKernelGGL(assign_resident_kernel<false>, dim3((unsigned)(units * wpu)), dim3(kAsResWaves * 64), lds,
                         s, k_tok, capacity, row0, count, cdir, K, assign, clu_stride, first, wpu, tpw, invn,
                         assign16, stride16);
    return hipGetLastError();
  }
  if (invn != nullptr) {  // the chunked kernel does not hold whole rows: a separate pass
    const hipError_t e = launch_inv_norm(k_tok, capacity, row0 - first, first, count, invn, clu_stride, units, s);
    if (e != hipSuccess) return e;
  }
  const int tiles = (count + kAsRows - 1) / kAsRows;
  hipLaunchKernelGGL(assign_kernel, dim3((unsigned)(units * tiles)), dim3(256), 0, s, k_tok,
                     capacity, row0, count, cdir, K, assign, clu_stride, first, tiles);
  return hipGetLastError();
}

hipError_t launch_index(const int32_t* assign, int clu_stride, int count, int K, int n_sink, int32_t* perm,
                        int32_t* offsets, int units, hipStream_t s) {
  if (K < 1 || K > kMaxClusters || count < 0) return hipErrorInvalidValue;
  const int ranges = index_ranges(units, K);
  const int stage = index_stage_ints(K, ranges, count);
  const size_t lds = ((size_t)index_fixed_ints(K, ranges) + stage) * sizeof(int);
  static std::once_flag lds_once;  // above the default dynamic LDS limit
  static hipError_t lds_status = hipSuccess;
  std::call_once(lds_once, [] {
    lds_status =
        hipFuncSetAttribute((const void*)index_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kIdxLdsMax);
  });
  if (lds_status != hipSuccess) return lds_status;
  const int xcd_map = (units % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(index_kernel, dim3((unsigned)(units * ranges)), dim3(kIdxThreads), lds, s, assign, clu_stride,
                     count, K, ranges, stage, xcd_map, n_sink, perm, offsets);
  return hipGetLastError();
}

hipError_t launch_delta(const uint16_t* cur_lab, const uint16_t* prev_lab, int stride16, int clu_stride, int count,
                        int K, const uint16_t* k_tok, int capacity, int n_sink, const double* invn, double* csum,
                        int32_t* csize, uint16_t* cdir, int units, hipStream_t s) {
  if ((stride16 & 1) != 0 || stride16 < count) return hipErrorInvalidValue;
  if (!delta_supported(K, count, units) || prev_lab == nullptr) return hipErrorInvalidValue;
  const int D = delta_dims(K);
  const int ranges = delta_ranges(units, K);
  const size_t lds = delta_lds_bytes(K, ranges);
  static std::once_flag lds_once;  // above the default dynamic LDS limit
  static hipError_t lds_status = hipSuccess;
  std::call_once(lds_once, [] {
    const void* fns[] = {(const void*)delta_kernel<32>, (const void*)delta_kernel<16>};
    for (const void* f : fns)
      if (lds_status == hipSuccess)
        lds_status = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kIdxLdsMax);
  });
  if (lds_status != hipSuccess) return lds_status;
  const int xcd_map = (units % 8 == 0) ? 1 : 0;
  const int fbits = delta_fbits(count);
  long long* sfix = reinterpret_cast<long long*>(csum);
  const dim3 grid((unsigned)(units * (kHeadDim / D) * ranges));
  if (D == 32)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(delta_kernel<32>), grid, dim3(kDelThreads), lds, s, cur_lab, prev_lab,
                       stride16, clu_stride, count, K, ranges, xcd_map, k_tok, capacity, n_sink, invn, fbits, sfix,
                       csize);
  else
    hipLaunchKernelGGL(HIP_KERNEL_NAME(delta_kernel<16>), grid, dim3(kDelThreads), lds, s, cur_lab, prev_lab,
                       stride16, clu_stride, count, K, ranges, xcd_map, k_tok, capacity, n_sink, invn, fbits, sfix,
                       csize);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long rows = (long)units * K;
  hipLaunchKernelGGL(delta_dirs_kernel, dim3((unsigned)((rows + 63) / 64)), dim3(1024), 0, s, sfix, csize, cdir, rows,
                     fbits);
  return hipGetLastError();
}

hipError_t launch_inv_norm(const uint16_t* k_tok, int capacity, int n_sink, int first, int count,
                           double* invn, int clu_stride, int units, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int blocks = (count + 16 * kNormRows - 1) / (16 * kNormRows);
  hipLaunchKernelGGL(inv_norm_kernel, dim3((unsigned)(units * blocks)), dim3(256), 0, s, k_tok, capacity,
                     n_sink, first, count, invn, clu_stride, blocks);
  return hipGetLastError();
}

hipError_t launch_update(int mode, const uint16_t* k_tok, const uint16_t* v_tok, int capacity, int n_sink,
                         const int32_t* perm, int clu_stride, const int32_t* offsets, int K,
                         const double* invn, double* csum, double* msum, float* cmean, int32_t* csize,
                         uint16_t* cdir, uint16_t* k_dst, uint16_t* v_dst, int units, hipStream_t s, int count) {
  const long waves = (long)units * K;
  const int fbits = mode == kUpdFixed ? delta_fbits(count) : 0;
  const dim3 grid((unsigned)((waves + 3) / 4));
#define CKV_UPD(M, O)                                                                                     \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(update_kernel<M, O>), grid, dim3(256), 0, s, k_tok, v_tok, capacity, \
                     n_sink, perm, clu_stride, offsets, K, invn, csum, msum, cmean, csize, cdir, k_dst, v_dst, \
                     units, fbits)
  if (invn == nullptr) {  // norms from the rows themselves: the final mode only
    if (mode != kUpdFinal) return hipErrorInvalidValue;
    CKV_UPD(kUpdFinal, true);
  } else if (mode == kUpdIter) {
    CKV_UPD(kUpdIter, false);
  } else if (mode == kUpdFixed) {
    CKV_UPD(kUpdFixed, false);
  } else if (mode == kUpdFinal) {
    CKV_UPD(kUpdFinal, false);
  } else {
    CKV_UPD(kUpdIncr, false);
  }
#undef CKV_UPD
  return hipGetLastError();
}

hipError_t launch_split(const uint16_t* k_clu, int n_sink, const int32_t* perm, int clu_stride,
                        const int32_t* offsets, int K, const double* csum, const int32_t* csize,
                        const uint16_t* cdir, double threshold, int32_t* plan, int32_t* assign, int units,
                        hipStream_t s) {
  if (K > kSplitMaxK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_plan_kernel, dim3((unsigned)units), dim3(kSplitWaves * 64), 0, s, K, csum, csize,
                     threshold, plan);
  hipLaunchKernelGGL(split_move_kernel, dim3((unsigned)units, (unsigned)kSplitPar), dim3(kSplitMoveWaves * 64), 0, s,
                     k_clu, n_sink, perm, clu_stride, offsets, K, cdir, plan, assign);
  return hipGetLastError();
}

}  // namespace ckv
