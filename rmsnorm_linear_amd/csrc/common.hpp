// Shared device helpers for the gfx950 kernels: vector types, bf16 bit
// conversions and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// float -> bf16 bits, round to nearest, ties to even (finite and inf; NaN kept NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Sum of squares of the 8 bf16 values in a 16-byte fragment, added to acc
// with float32 fused multiply-adds (each bf16 widens exactly to float32).
__device__ __forceinline__ float sumsq_bf16x8(const u32x4& v, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_lo(v[i]);
    const float hi = bf16_hi(v[i]);
    acc = fmaf(lo, lo, acc);
    acc = fmaf(hi, hi, acc);
  }
  return acc;
}

// LayerNorm statistics of 8 bf16 values, shifted by the row's value `sh`:
// s1 += sum (x - sh), s2 += sum (x - sh)^2.  The shift keeps the variance
// sum2/K - (sum1/K)^2 free of cancellation when the row mean is large
// against its spread.
__device__ __forceinline__ void lnstat_bf16x8(const u32x4& v, float sh, float& s1, float& s2) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_lo(v[i]) - sh;
    const float hi = bf16_hi(v[i]) - sh;
    s1 += lo;
    s2 = fmaf(lo, lo, s2);
    s1 += hi;
    s2 = fmaf(hi, hi, s2);
  }
}

// Butterfly sum over lanes that differ in the bits of `mask_bits` (xor).
template <int MASK>
__device__ __forceinline__ float xor_sum(float v) {
  return v + __shfl_xor(v, MASK, kWave);
}

__device__ __forceinline__ float silu(float t) { return t / (1.0f + __expf(-t)); }

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  // Workgroups are dealt round-robin to the 8 XCDs (bid % 8).  Give each XCD
  // a contiguous run of the logical tile order so neighbouring tiles, which
  // share operand panels, land in the same L2.
  const int nx = 8;
  int per = nblocks / nx;
  if (bid >= per * nx) return bid;  // ragged tail keeps its slot
  return (bid % nx) * per + bid / nx;
}

}  // namespace fn
