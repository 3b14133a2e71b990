// Bandwidth-bound kernels: the offline weight fold, the unfused baseline's
// RMSNorm, the two-stream variant's row-scale and post-scale, and a fill.
// All use 16-byte (or 8-byte) vector accesses with consecutive lanes on
// consecutive addresses so every wavefront access covers whole 128-byte
// lines.

#include "common.hpp"
#include "kernels.hpp"

namespace fn {

namespace {

constexpr int kRowThreads = 256;

// float64 -> bf16 bits with a single round to nearest even.  The float64
// value is first rounded to float32 *to odd* (truncate, then set the last
// bit if anything was dropped); a float32 rounded to odd carries enough
// extra bits that rounding it to bf16 (nearest even) gives the same result
// as rounding the float64 value directly (Boldo and Melquiond, "Emulation of
// FMA and correctly rounded sums: proved algorithms using rounding to odd").
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double p) {
  float f = (float)p;  // nearest even
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != p && p == p) {
    if (fabs(back) > fabs(p)) u -= 1u;  // went away from zero: step back (sign-magnitude)
    u |= 1u;
  }
  return f32_to_bf16_bits(__uint_as_float(u));
}

template <int WDT, int ODT>
__global__ void fold_kernel(const void* __restrict__ W, const float* __restrict__ g, int64_t groups, int K,
                            void* __restrict__ out) {
  // one group = 4 consecutive elements of a row (K % 4 == 0)
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < groups;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = q * 4;
    const int k0 = (int)(e0 % K);
    const float4 gg = *reinterpret_cast<const float4*>(g + k0);
    float w[4];
    if constexpr (WDT == 0) {
      const float4 v = reinterpret_cast<const float4*>(W)[q];
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      const uint2 v = reinterpret_cast<const uint2*>(W)[q];
      w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
    }
    const float gv[4] = {gg.x, gg.y, gg.z, gg.w};
    double prod[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) prod[i] = (double)w[i] * (double)gv[i];  // exact
    if constexpr (ODT == 0) {
      float4 o;
      o.x = (float)prod[0]; o.y = (float)prod[1]; o.z = (float)prod[2]; o.w = (float)prod[3];
      reinterpret_cast<float4*>(out)[q] = o;
    } else {
      uint2 o;
      o.x = f64_to_bf16_bits(prod[0]) | (f64_to_bf16_bits(prod[1]) << 16);
      o.y = f64_to_bf16_bits(prod[2]) | (f64_to_bf16_bits(prod[3]) << 16);
      reinterpret_cast<uint2*>(out)[q] = o;
    }
  }
}

// Block-wide sum over kRowThreads threads.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = xor_sum<1>(v); v = xor_sum<2>(v); v = xor_sum<4>(v);
  v = xor_sum<8>(v); v = xor_sum<16>(v); v = xor_sum<32>(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kRowThreads / 64; ++i) t += red[i];
  return t;
}

// Loads 4 consecutive elements of a row as float.
template <int DT>
__device__ __forceinline__ void load4(const void* base, int64_t idx4, float v[4]) {
  if constexpr (DT == 0) {
    const float4 f = reinterpret_cast<const float4*>(base)[idx4];
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    const uint2 u = reinterpret_cast<const uint2*>(base)[idx4];
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
  }
}

template <int DT>
__device__ float row_sumsq(const void* x, int64_t row, int K) {
  float acc = 0.f;
  const int64_t base4 = row * (K / 4);
  for (int c = threadIdx.x; c < K / 4; c += kRowThreads) {
    float v[4];
    load4<DT>(x, base4 + c, v);
    acc += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  return acc;
}

template <int DT>
__global__ __launch_bounds__(kRowThreads) void rmsnorm_kernel(const void* __restrict__ x,
                                                              const float* __restrict__ g, int K, float eps,
                                                              void* __restrict__ xn) {
  __shared__ float red[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const float ss = block_sum(row_sumsq<DT>(x, row, K), red);
  const float s = rsqrtf(ss / (float)K + eps);
  const int64_t base4 = row * (K / 4);
  for (int c = threadIdx.x; c < K / 4; c += kRowThreads) {
    float v[4];
    load4<DT>(x, base4 + c, v);
    const float4 gg = reinterpret_cast<const float4*>(g)[c];
    const float o0 = v[0] * s * gg.x, o1 = v[1] * s * gg.y, o2 = v[2] * s * gg.z, o3 = v[3] * s * gg.w;
    if constexpr (DT == 0) {
      reinterpret_cast<float4*>(xn)[base4 + c] = make_float4(o0, o1, o2, o3);
    } else {
      uint2 u;
      u.x = pack_bf16x2(o0, o1);
      u.y = pack_bf16x2(o2, o3);
      reinterpret_cast<uint2*>(xn)[base4 + c] = u;
    }
  }
}

template <int DT>
__global__ __launch_bounds__(kRowThreads) void row_scale_kernel(const void* __restrict__ x, int K, float eps,
                                                                float* __restrict__ s) {
  __shared__ float red[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const float ss = block_sum(row_sumsq<DT>(x, row, K), red);
  if (threadIdx.x == 0) s[row] = rsqrtf(ss / (float)K + eps);
}

template <int ODT>
__global__ void post_scale_kernel(const float* __restrict__ z, const float* __restrict__ s, int64_t groups,
                                  int N, void* __restrict__ y) {
  // one group = 4 consecutive outputs of a row (N % 4 == 0)
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < groups;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = (q * 4) / N;
    const float sc = s[row];
    const float4 v = reinterpret_cast<const float4*>(z)[q];
    if constexpr (ODT == 0) {
      reinterpret_cast<float4*>(y)[q] = make_float4(v.x * sc, v.y * sc, v.z * sc, v.w * sc);
    } else {
      uint2 u;
      u.x = pack_bf16x2(v.x * sc, v.y * sc);
      u.y = pack_bf16x2(v.z * sc, v.w * sc);
      reinterpret_cast<uint2*>(y)[q] = u;
    }
  }
}

__global__ void fill_kernel(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// One thread per (position, pair): the angle p * base^(-2i/d) and its
// cosine and sine in float64 (the definition of the rotary embedding in
// RoFormer: Enhanced Transformer with Rotary Position Embedding, Section 3.2),
// each rounded once to float32.
__global__ void rope_table_kernel(double log2_base, int half, int64_t n, float2* __restrict__ t) {
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = q / half;
    const int i = (int)(q % half);
    const double theta = exp2(-(double)i / (double)half * log2_base);
    const double a = (double)p * theta;
    t[q] = make_float2((float)cos(a), (float)sin(a));
  }
}

int grid_for(int64_t work, int threads) {
  int64_t b = (work + threads - 1) / threads;
  const int64_t cap = 256 * 16;  // enough resident waves to saturate HBM
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

hipError_t launch_fold(const void* W, int w_dt, const float* g, int64_t N, int64_t K, void* Ws, int out_dt,
                       hipStream_t st) {
  const int64_t groups = N * K / 4;
  const int threads = 256;
  const int grid = grid_for(groups, threads);
  const int k = (int)K;
  if (w_dt == 0 && out_dt == 0) hipLaunchKernelGGL((fold_kernel<0, 0>), dim3(grid), dim3(threads), 0, st, W, g, groups, k, Ws);
  else if (w_dt == 0 && out_dt == 1) hipLaunchKernelGGL((fold_kernel<0, 1>), dim3(grid), dim3(threads), 0, st, W, g, groups, k, Ws);
  else if (w_dt == 1 && out_dt == 0) hipLaunchKernelGGL((fold_kernel<1, 0>), dim3(grid), dim3(threads), 0, st, W, g, groups, k, Ws);
  else hipLaunchKernelGGL((fold_kernel<1, 1>), dim3(grid), dim3(threads), 0, st, W, g, groups, k, Ws);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const void* x, int dt, const float* g, int64_t M, int64_t K, float eps, void* xn,
                          hipStream_t st) {
  if (dt == 0) hipLaunchKernelGGL((rmsnorm_kernel<0>), dim3((unsigned)M), dim3(kRowThreads), 0, st, x, g, (int)K, eps, xn);
  else hipLaunchKernelGGL((rmsnorm_kernel<1>), dim3((unsigned)M), dim3(kRowThreads), 0, st, x, g, (int)K, eps, xn);
  return hipGetLastError();
}

hipError_t launch_row_scale(const void* x, int dt, int64_t M, int64_t K, float eps, float* s, hipStream_t st) {
  if (dt == 0) hipLaunchKernelGGL((row_scale_kernel<0>), dim3((unsigned)M), dim3(kRowThreads), 0, st, x, (int)K, eps, s);
  else hipLaunchKernelGGL((row_scale_kernel<1>), dim3((unsigned)M), dim3(kRowThreads), 0, st, x, (int)K, eps, s);
  return hipGetLastError();
}

hipError_t launch_post_scale(const float* z, const float* s, int64_t M, int64_t N, void* y, int y_dt,
                             hipStream_t st) {
  const int64_t groups = M * N / 4;
  const int grid = grid_for(groups, 256);
  if (y_dt == 0) hipLaunchKernelGGL((post_scale_kernel<0>), dim3(grid), dim3(256), 0, st, z, s, groups, (int)N, y);
  else hipLaunchKernelGGL((post_scale_kernel<1>), dim3(grid), dim3(256), 0, st, z, s, groups, (int)N, y);
  return hipGetLastError();
}

hipError_t launch_rope_table(double base, int rot_dim, int64_t n_pos, float* t, hipStream_t st) {
  const int half = rot_dim / 2;
  const int64_t n = n_pos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, log2(base), half, n,
                     reinterpret_cast<float2*>(t));
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* p, uint32_t value, int64_t n_words, hipStream_t st) {
  const int grid = grid_for(n_words, 256);
  hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(256), 0, st, static_cast<uint32_t*>(p), value, n_words);
  return hipGetLastError();
}

}  // namespace fn
