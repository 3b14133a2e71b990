// float32 norm-then-project: v_mfma_f32_16x16x4_f32 contraction of x with
// the folded W*, row sum of squares from the same A operands, deferred row
// scale in the epilogue (FlashNorm Abstract, points (i) and (ii)).
//
// Workgroup tile 32 x 64, K step 32, 4 waves as 2 x 2, each wave a 16 x 32
// block (two MFMA tiles).  Operands go through LDS with rows padded to 36
// floats.

#include "common.hpp"
#include "kernels.hpp"

namespace fn {

namespace {

constexpr int BM = 32, BN = 64, BK = 32, LD = BK + 4;

template <bool SUMSQ>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmF32Args p) {
  __shared__ float As[BM * LD];
  __shared__ float Bs[BN * LD];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 15, fk = lane >> 4;
  const int M = p.M, K = p.K, N = p.N;
  const int tiles_n = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM;
  const int n0 = (blockIdx.x % tiles_n) * BN;

  // loader coordinates: a 32-float K slice is 8 float4
  const int lr = tid >> 3, lc = (tid & 7) * 4;
  const float* a_src = p.A + (size_t)min(m0 + lr, M - 1) * K + lc;
  const float* b_src0 = p.B + (size_t)min(n0 + lr, N - 1) * K + lc;
  const float* b_src1 = p.B + (size_t)min(n0 + 32 + lr, N - 1) * K + lc;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool ok = k0 + lc < K;
    const float4 va = ok ? *reinterpret_cast<const float4*>(a_src + k0) : z4;
    const float4 vb0 = ok ? *reinterpret_cast<const float4*>(b_src0 + k0) : z4;
    const float4 vb1 = ok ? *reinterpret_cast<const float4*>(b_src1 + k0) : z4;
    __syncthreads();
    *reinterpret_cast<float4*>(&As[lr * LD + lc]) = va;
    *reinterpret_cast<float4*>(&Bs[lr * LD + lc]) = vb0;
    *reinterpret_cast<float4*>(&Bs[(32 + lr) * LD + lc]) = vb1;
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 4) {
      const float a = As[(wm * 16 + frow) * LD + ks + fk];
      const float b0 = Bs[(wn * 32 + frow) * LD + ks + fk];
      const float b1 = Bs[(wn * 32 + 16 + frow) * LD + ks + fk];
      if constexpr (SUMSQ) ss = fmaf(a, a, ss);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b1, acc1, 0, 0, 0);
    }
  }
  float srow[4];
  if constexpr (SUMSQ) {
    ss = xor_sum<16>(ss);
    ss = xor_sum<32>(ss);
    const float s = rsqrtf(ss * p.inv_k + p.eps);
#pragma unroll
    for (int r = 0; r < 4; ++r) srow[r] = __shfl(s, 4 * fk + r, kWave);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) srow[r] = 1.0f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + wm * 16 + 4 * fk + r;
    const int n = n0 + wn * 32 + frow;
    if (m < M) {
      if (n < N) p.Y[(size_t)m * N + n] = acc0[r] * srow[r];
      if (n + 16 < N) p.Y[(size_t)m * N + n + 16] = acc1[r] * srow[r];
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(bool sumsq, const GemmF32Args& a, hipStream_t st) {
  const int grid = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (sumsq) hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace fn
