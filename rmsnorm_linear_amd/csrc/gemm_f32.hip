// float32 norm-then-project: v_mfma_f32_16x16x4_f32 contraction of x with
// the folded W*, row sum of squares from the same A operands, deferred row
// scale in the epilogue (FlashNorm Abstract, points (i) and (ii)); the
// LayerNorm epilogue also keeps shifted row sums of x and subtracts
// mean * (column sum of W*) before the scale.
//
// The float32 workloads are small (a SmolLM2 layer: 0.14 GFLOP), so the
// kernel is built for latency, not for reuse: no LDS staging of operands.
// Workgroup tile 16 (rows of x) x 32 (rows of W*), eight waves that split K:
// wave w takes the 16-wide K steps s with s % 8 == w, loading its operands
// straight from memory in 16-byte pieces, several steps ahead.  A lane's
// float4 covers four consecutive k; MFMA j of a step takes element j of
// every lane, so the four MFMAs of a step together cover its 16 k values
// (the same k permutation on both operands leaves the sum unchanged).  The
// eight partial results meet in LDS, and wave t finishes output subtile t.

#include "common.hpp"
#include "kernels.hpp"

namespace fn {

namespace {

constexpr int BM = 16, BN = 32, KS = 16;

template <int EPI, bool SUMSQ, int kWaves, int kUnroll>
__global__ __launch_bounds__(kWaves * 64) void gemm_f32_kernel(GemmF32Args p) {
  static_assert(kWaves >= BN / 16, "one output subtile per wave in the epilogue");
  constexpr bool LNS = (EPI == EPI_LN) && SUMSQ;  // LayerNorm statistics
  __shared__ f32x4 red[kWaves][BN / 16][64];
  __shared__ float red_ss[kWaves][64];
  __shared__ float red_s1[LNS ? kWaves : 1][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int frow = lane & 15, fk = lane >> 4;
  const int M = p.M, K = p.K, N = p.N;
  const int tiles_n = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM;
  const int n0 = (blockIdx.x % tiles_n) * BN;

  // operand rows of this lane (clamped: rows past the end are read, never stored)
  const float* a_src = p.A + (size_t)min(m0 + frow, M - 1) * K + 4 * fk;
  const float* b_src[BN / 16];
#pragma unroll
  for (int t = 0; t < BN / 16; ++t) b_src[t] = p.B + (size_t)min(n0 + 16 * t + frow, N - 1) * K + 4 * fk;

  f32x4 acc[BN / 16];
#pragma unroll
  for (int t = 0; t < BN / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  // LayerNorm: sums of x - sh and (x - sh)^2, sh = the row's first element
  float s1 = 0.f;
  const float sh = LNS ? p.A[(size_t)min(m0 + frow, M - 1) * K] : 0.f;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const int steps = (K + KS - 1) / KS;
  for (int s0 = wave; s0 < steps; s0 += kWaves * kUnroll) {
    f32x4 a[kUnroll], b[kUnroll][BN / 16];
    bool aok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = (s0 + u * kWaves) * KS;
      const bool ok = (s0 + u * kWaves < steps) && (k + 4 * fk < K);  // K % 4 == 0: whole float4s
      aok[u] = ok;
      a[u] = ok ? *reinterpret_cast<const f32x4*>(a_src + k) : z4;
#pragma unroll
      for (int t = 0; t < BN / 16; ++t) b[u][t] = ok ? *reinterpret_cast<const f32x4*>(b_src[t] + k) : z4;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (LNS) {
          if (aok[u]) {  // float4s past K (zeros) must not count
            const float d = a[u][j] - sh;
            s1 += d;
            ss = fmaf(d, d, ss);
          }
        } else if constexpr (SUMSQ) {
          ss = fmaf(a[u][j], a[u][j], ss);
        }
#pragma unroll
        for (int t = 0; t < BN / 16; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][j], b[u][t][j], acc[t], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int t = 0; t < BN / 16; ++t) red[wave][t][lane] = acc[t];
  red_ss[wave][lane] = ss;
  if constexpr (LNS) red_s1[wave][lane] = s1;
  __syncthreads();

  // wave t: output subtile t (columns n0 + 16 t ...)
  if (wave >= BN / 16) return;
  const int t = wave;
  f32x4 c = red[0][t][lane];
  float q = red_ss[0][lane];
  float q1 = LNS ? red_s1[0][lane] : 0.f;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    c += red[w][t][lane];
    q += red_ss[w][lane];
    if constexpr (LNS) q1 += red_s1[w][lane];
  }
  // accumulator layout: lane holds rows 4 (lane / 16) + r, column lane % 16;
  // the row sum of squares of row i sits in lanes with lane % 16 == i
  float srow[4], mrow[4];
  if constexpr (LNS) {
    q = xor_sum<32>(xor_sum<16>(q));
    q1 = xor_sum<32>(xor_sum<16>(q1));
    const float md = q1 * p.inv_k;  // lane i (< 16) holds row i's sums and shift
    const float sc = rsqrtf(fmaxf(fmaf(-md, md, q * p.inv_k), 0.f) + p.eps);
    const float mu = sh + md;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      srow[r] = __shfl(sc, 4 * fk + r, kWave);
      mrow[r] = __shfl(mu, 4 * fk + r, kWave);
    }
  } else if constexpr (SUMSQ) {
    q = xor_sum<16>(q);
    q = xor_sum<32>(q);
    const float sc = rsqrtf(q * p.inv_k + p.eps);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      srow[r] = __shfl(sc, 4 * fk + r, kWave);
      mrow[r] = 0.f;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      srow[r] = 1.0f;
      mrow[r] = 0.f;
    }
  }
  const int n = n0 + 16 * t + frow;
  float cn = 0.f, bn = 0.f;
  if constexpr (EPI == EPI_LN) {
    if (n < N) {
      if constexpr (LNS) cn = p.ln_c[n];
      if (p.ln_b != nullptr) bn = p.ln_b[n];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + 4 * fk + r;
    if (m < M && n < N) {
      if constexpr (EPI == EPI_LN)
        p.Y[(size_t)m * N + n] = fmaf(fmaf(-mrow[r], cn, c[r]), srow[r], bn);
      else
        p.Y[(size_t)m * N + n] = c[r] * srow[r];
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(int epi, bool sumsq, const GemmF32Args& a, hipStream_t st) {
  // 16 x 32 tiles (240 workgroups on the SmolLM2 shape), eight waves, three
  // steps in flight each: 6.7 us of kernel time there, against 10.6 us for
  // 16 x 64 tiles with four waves, 7.4 us for 16 x 32 with four, 7.3 us for
  // 16 x 16 with eight, 6.8 us with all of a wave's steps in flight.
  constexpr int W = 8, U = 3;
  const int grid = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (epi == EPI_PLAIN) {
    if (sumsq) hipLaunchKernelGGL((gemm_f32_kernel<EPI_PLAIN, true, W, U>), dim3(grid), dim3(W * 64), 0, st, a);
    else hipLaunchKernelGGL((gemm_f32_kernel<EPI_PLAIN, false, W, U>), dim3(grid), dim3(W * 64), 0, st, a);
  } else if (epi == EPI_LN) {
    if (sumsq) hipLaunchKernelGGL((gemm_f32_kernel<EPI_LN, true, W, U>), dim3(grid), dim3(W * 64), 0, st, a);
    else hipLaunchKernelGGL((gemm_f32_kernel<EPI_LN, false, W, U>), dim3(grid), dim3(W * 64), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fn
