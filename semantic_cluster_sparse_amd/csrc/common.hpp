// Device helpers shared by the libckv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckv {

constexpr int kHeadDim = 128;
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> f32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f64 -> bf16 bit pattern, round to nearest with ties to the even significand,
// directly from f64 (no intermediate f32 rounding).  The quantum of the
// result is 2^(max(e,-126)-7) for a magnitude with binary exponent e.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  const unsigned long long bits = (unsigned long long)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(bits >> 63) << 15;
  const int biased = (int)((bits >> 52) & 0x7FF);
  if (biased == 0x7FF) {
    return (bits & 0xFFFFFFFFFFFFFull) ? (uint16_t)0x7FC0 : (uint16_t)(sign | 0x7F80);
  }
  const double a = fabs(x);
  if (a == 0.0) return (uint16_t)sign;
  int e = biased - 1023;           // subnormal doubles land far below bf16 range
  if (e < -126) e = -126;
  const double r = rint(a * ldexp(1.0, 7 - e)) * ldexp(1.0, e - 7);  // exact scalings
  const double kMax = 3.3895313892515355e38;                         // (2 - 2^-7) * 2^127
  if (r > kMax) return (uint16_t)(sign | 0x7F80);
  return (uint16_t)(sign | (__float_as_uint((float)r) >> 16));
}

// Wait until every vector memory operation this wave has issued is complete
// (on gfx9 vmcnt counts stores too, so stores are acknowledged by the memory
// side), and keep the compiler from moving any memory access across this
// point.  A workgroup runs it before moving a device-scope arrival counter,
// so its agent-scope stores (which write through to the coherence point) are
// visible to whichever workgroup sees the counter's final value.
__device__ __forceinline__ void drain_memory_ops() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}

// Lane id within the wave.
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Butterfly sum across the lanes that differ only in the bits of `mask_bits`
// (each xor step in turn).  Uses ds_bpermute through __shfl_xor.
template <typename T>
__device__ __forceinline__ T xor_sum16(T v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

// DPP move within rows of 16 lanes (gfx9 dpp_ctrl encodings).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within 16

// Sum over each row of 16 lanes; every lane of the row gets the same
// (bitwise identical) value because each step adds commutative pairs.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}

// DPP move of an int with explicit row / bank masks; lanes whose source is
// outside the row (or rows not in row_mask) read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum across the 64 lanes of a wave (DPP row shifts, then
// row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i32<0x111, 0xF>(v);  // row_shr:1
  v += dpp_i32<0x112, 0xF>(v);  // row_shr:2
  v += dpp_i32<0x114, 0xF>(v);  // row_shr:4
  v += dpp_i32<0x118, 0xF>(v);  // row_shr:8
  v += dpp_i32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_i32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

template <int CTRL>
__device__ __forceinline__ int dpp_row_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Bitwise AND / OR over the 64 lanes of a wave (DPP within rows of 16, then
// the four row results through readlane); the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  int x = (int)v;
  x &= __builtin_amdgcn_mov_dpp(x, kDppXor1, 0xF, 0xF, true);
  x &= __builtin_amdgcn_mov_dpp(x, kDppXor2, 0xF, 0xF, true);
  x &= __builtin_amdgcn_mov_dpp(x, kDppHalfMirror, 0xF, 0xF, true);
  x &= __builtin_amdgcn_mov_dpp(x, kDppMirror, 0xF, 0xF, true);
  return (uint32_t)(__builtin_amdgcn_readlane(x, 0) & __builtin_amdgcn_readlane(x, 16) &
                    __builtin_amdgcn_readlane(x, 32) & __builtin_amdgcn_readlane(x, 48));
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  int x = (int)v;
  x |= __builtin_amdgcn_mov_dpp(x, kDppXor1, 0xF, 0xF, true);
  x |= __builtin_amdgcn_mov_dpp(x, kDppXor2, 0xF, 0xF, true);
  x |= __builtin_amdgcn_mov_dpp(x, kDppHalfMirror, 0xF, 0xF, true);
  x |= __builtin_amdgcn_mov_dpp(x, kDppMirror, 0xF, 0xF, true);
  return (uint32_t)(__builtin_amdgcn_readlane(x, 0) | __builtin_amdgcn_readlane(x, 16) |
                    __builtin_amdgcn_readlane(x, 32) | __builtin_amdgcn_readlane(x, 48));
}

// Exclusive prefix sum over a block of `nthreads` threads (nthreads <= 1024,
// multiple of 64).  `scratch` needs nthreads/64 + 1 ints of LDS.  Returns the
// exclusive prefix of `v` and writes the block total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int nwaves = (blockDim.x + kWave - 1) / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) scratch[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) {
      int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[nwaves] = run;
  }
  __syncthreads();
  const int excl = scratch[wave] + x - v;
  *total = scratch[nwaves];
  __syncthreads();
  return excl;
}

}  // namespace ckv
