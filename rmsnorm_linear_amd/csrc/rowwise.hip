// Bandwidth-bound kernels: the offline weight folds (RMSNorm and LayerNorm),
// the unfused baselines' RMSNorm and LayerNorm, the two-stream variant's
// row-scale and post-scale, the rotary table, the fp8 weight quantiser, the
// MLA latent norms, and a fill.
// All use 16-byte (or 8-byte) vector accesses with consecutive lanes on
// consecutive addresses so every wavefront access covers whole 128-byte
// lines.

#include <algorithm>

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

// Block-wide float64 sum over kRowThreads threads.
__device__ __forceinline__ double block_sum_d(double v, double* red) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, kWave);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kRowThreads / 64; ++i) t += red[i];
  return t;
}

// LayerNorm fold, one workgroup per weight row n: W*[n,k] = round(g[k]
// W[n,k]) as fold_kernel does, c[n] = sum of the stored W*[n,k], b[n] =
// sum_k beta[k] W[n,k] + bias[n].  Both sums run in float64 (the products
// are exact there) and are rounded once to float32.  Each thread writes
// only the elements it read, so W* may alias W.
template <int WDT, int ODT>
__global__ __launch_bounds__(kRowThreads) void fold_layernorm_kernel(const void* W,
                                                                     const float* __restrict__ g,
                                                                     const float* __restrict__ beta,
                                                                     const float* __restrict__ bias, int K,
                                                                     void* Ws, float* __restrict__ c,
                                                                     float* __restrict__ b) {
  __shared__ double red_c[kRowThreads / 64], red_b[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const int64_t base4 = row * (K / 4);
  double sc = 0.0, sb = 0.0;
  for (int q = threadIdx.x; q < K / 4; q += kRowThreads) {
    float w[4];
    load4<WDT>(W, base4 + q, w);
    const float4 gg = reinterpret_cast<const float4*>(g)[q];
    const float gv[4] = {gg.x, gg.y, gg.z, gg.w};
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (beta) {
      const float4 t = reinterpret_cast<const float4*>(beta)[q];
      bv[0] = t.x; bv[1] = t.y; bv[2] = t.z; bv[3] = t.w;
    }
    double prod[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      prod[i] = (double)w[i] * (double)gv[i];  // exact
      sb += (double)bv[i] * (double)w[i];      // exact product
    }
    if constexpr (ODT == 0) {
      float4 o;
      o.x = (float)prod[0]; o.y = (float)prod[1]; o.z = (float)prod[2]; o.w = (float)prod[3];
      sc += ((double)o.x + (double)o.y) + ((double)o.z + (double)o.w);
      reinterpret_cast<float4*>(Ws)[base4 + q] = o;
    } else {
      uint2 o;
      o.x = f64_to_bf16_bits(prod[0]) | (f64_to_bf16_bits(prod[1]) << 16);
      o.y = f64_to_bf16_bits(prod[2]) | (f64_to_bf16_bits(prod[3]) << 16);
      sc += ((double)bf16_lo(o.x) + (double)bf16_hi(o.x)) + ((double)bf16_lo(o.y) + (double)bf16_hi(o.y));
      reinterpret_cast<uint2*>(Ws)[base4 + q] = o;
    }
  }
  const double tc = block_sum_d(sc, red_c);
  const double tb = block_sum_d(sb, red_b);
  if (threadIdx.x == 0) {
    c[row] = (float)tc;
    b[row] = (float)(tb + (bias ? (double)bias[row] : 0.0));
  }
}

// ---- row kernels: one wave per row ----------------------------------------
// The unfused baselines' RMSNorm and LayerNorm (normalised rows written in
// the input dtype) and the row statistics alone (scale, and for LayerNorm
// the mean) for the two-stream variant and the fused variant's statistics
// pass.  Workgroups of four waves: with many rows, one wave per row (four
// rows per workgroup, sums meet by butterfly within the wave, no barrier);
// with few rows, all four waves on one row (the four partial sums meet in
// LDS).  Lanes read the row in 16-byte pieces (8 bf16 or 4 float32),
// several in flight.  LayerNorm
// sums are shifted by the row's first element (x - x[0] and its square),
// which keeps the variance sum2/K - (sum1/K)^2 free of cancellation.
constexpr int kRowsPerBlock = 4;

enum RowOp { ROW_SCALE = 0, ROW_LN_STATS = 1, ROW_RMSNORM = 2, ROW_LAYERNORM = 3 };

template <int DT>
__device__ __forceinline__ void unpack16(const u32x4& v, float* f) {
  if constexpr (DT == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(v[i]);
      f[2 * i + 1] = bf16_hi(v[i]);
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
  return xor_sum<32>(xor_sum<16>(xor_sum<8>(xor_sum<4>(xor_sum<2>(xor_sum<1>(v))))));
}

template <int DT, int OP, int WPR>
__global__ __launch_bounds__(kRowsPerBlock * 64) void row_kernel(const void* __restrict__ x, int64_t M, int K,
                                                                 float eps, const float* __restrict__ g,
                                                                 const float* __restrict__ beta,
                                                                 float* __restrict__ s_out, float* __restrict__ mu_out,
                                                                 void* __restrict__ xn) {
  static_assert(WPR == 1 || WPR == kRowsPerBlock, "one wave per row, or the whole workgroup");
  constexpr int E = DT == 0 ? 4 : 8;  // elements per 16-byte piece
  constexpr bool LN = OP == ROW_LN_STATS || OP == ROW_LAYERNORM;
  const int wave = threadIdx.x >> 6;
  const int lane = (WPR == 1) ? (threadIdx.x & 63) : threadIdx.x;  // position among the row's threads
  constexpr int STRIDE = 64 * WPR;
  const int64_t row = (WPR == 1) ? (int64_t)blockIdx.x * kRowsPerBlock + wave : (int64_t)blockIdx.x;
  if (row >= M) return;  // workgroup-uniform when WPR > 1
  const int C = K / E;  // 16-byte pieces per row
  const size_t row_bytes = (size_t)K * (DT == 0 ? 4 : 2);
  const u32x4* xr = reinterpret_cast<const u32x4*>(static_cast<const char*>(x) + row * row_bytes);
  float sh = 0.f;
  if constexpr (LN) {
    if constexpr (DT == 0)
      sh = static_cast<const float*>(x)[row * K];
    else
      sh = __uint_as_float((uint32_t) static_cast<const uint16_t*>(x)[row * K] << 16);
  }
  float a = 0.f, b = 0.f;  // RMS: a = sum x^2.  LayerNorm: a = sum (x - sh), b = sum (x - sh)^2
#pragma unroll 8
  for (int c = lane; c < C; c += STRIDE) {
    float f[E];
    unpack16<DT>(xr[c], f);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if constexpr (LN) {
        const float d = f[e] - sh;
        a += d;
        b = fmaf(d, d, b);
      } else {
        a = fmaf(f[e], f[e], a);
      }
    }
  }
  a = wave_sum(a);
  if constexpr (LN) b = wave_sum(b);
  if constexpr (WPR > 1) {
    __shared__ float red[2][WPR];
    if ((threadIdx.x & 63) == 0) {
      red[0][wave] = a;
      red[1][wave] = b;
    }
    __syncthreads();
    a = b = 0.f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) {
      a += red[0][w];
      b += red[1][w];
    }
  }
  float s, mu = 0.f;
  if constexpr (LN) {
    const float md = a / (float)K;
    mu = sh + md;
    s = rsqrtf(fmaxf(fmaf(-md, md, b / (float)K), 0.f) + eps);
  } else {
    s = rsqrtf(a / (float)K + eps);
  }
  if constexpr (OP == ROW_SCALE || OP == ROW_LN_STATS) {
    if (lane == 0) {
      s_out[row] = s;
      if constexpr (LN) mu_out[row] = mu;
    }
  } else {
    u32x4* out = reinterpret_cast<u32x4*>(static_cast<char*>(xn) + row * row_bytes);
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    const f32x4* b4 = reinterpret_cast<const f32x4*>(beta);
#pragma unroll 2
    for (int c = lane; c < C; c += STRIDE) {
      float f[E], o[E];
      unpack16<DT>(xr[c], f);
#pragma unroll
      for (int h = 0; h < E / 4; ++h) {
        const f32x4 gg = g4[c * (E / 4) + h];
        f32x4 bb = {0.f, 0.f, 0.f, 0.f};
        if (LN && beta != nullptr) bb = b4[c * (E / 4) + h];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = f[4 * h + e];
          o[4 * h + e] = LN ? fmaf((v - mu) * s, gg[e], bb[e]) : v * s * gg[e];
        }
      }
      u32x4 w;
      if constexpr (DT == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(o[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(o[2 * i], o[2 * i + 1]);
      }
      out[c] = w;
    }
  }
}

template <int OP>
hipError_t launch_rows(const void* x, int dt, int64_t M, int64_t K, float eps, const float* g, const float* beta,
                       float* s, float* mu, void* xn, hipStream_t st) {
  // one wave per row once there are rows for at least 8 waves per CU and
  // each lane has several 16-byte pieces of its row to read
  const int64_t pieces = K * (dt == 0 ? 4 : 2) / 16;
  const bool wave_rows = M >= 2048 && pieces >= 4 * 64;
  const dim3 block(kRowsPerBlock * 64);
  const dim3 grid((unsigned)(wave_rows ? (M + kRowsPerBlock - 1) / kRowsPerBlock : M));
#define FN_ROWS(D, W) hipLaunchKernelGGL((row_kernel<D, OP, W>), grid, block, 0, st, x, M, (int)K, eps, g, beta, s, mu, xn)
  if (dt == 0) {
    if (wave_rows) FN_ROWS(0, 1); else FN_ROWS(0, kRowsPerBlock);
  } else {
    if (wave_rows) FN_ROWS(1, 1); else FN_ROWS(1, kRowsPerBlock);
  }
#undef FN_ROWS
  return hipGetLastError();
}

// ---- fp8 (OCP E4M3) per-channel quantisation --------------------------------
// E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; largest finite
// 448, smallest normal 2^-6, subnormal spacing 2^-9; 0x7F is NaN.

// Round a float64 value to the nearest E4M3 value (ties to even) and return
// its code; beyond the largest finite value (from 464, the tie between 448
// and the unrepresentable 480) it saturates to 448.  NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_code_rne(double v) {
  const uint32_t sign = signbit(v) ? 0x80u : 0u;
  const double a = fabs(v);
  if (a != a) return sign | 0x7Fu;
  if (a >= 464.0) return sign | 0x7Eu;
  if (a < 0.015625) return sign | (uint32_t)rint(a * 512.0);  // multiples of 2^-9; 8 is the code of 2^-6
  int e = ilogb(a);                       // 2^e <= a < 2^(e+1), e in [-6, 8]
  double n = rint(ldexp(a, 3 - e));       // significand in units of 2^(e-3): 8 .. 16
  if (n == 16.0) {
    n = 8.0;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | ((uint32_t)n - 8u);
}

// The same rounding of |w| / q, exactly, in float32 arithmetic (q >= 2^-96,
// rq = float32(1 / q)).  t = |w| rq is within two float32 roundings of the
// quotient, so it falls in (or at the edge of) the gap between the two E4M3
// values that enclose the quotient.  For t >= 2^-6 the gap's lower end is t
// with all but its top three significand bits cleared (an E4M3 value has
// three), and its midpoint that value with the fourth bit set; below 2^-6
// (the subnormal values, spacing 2^-9, the spacing of [2^-6, 2^-5)) the
// same is done on t + 2^-6 and 2^-6 taken back off.  The sign of the exact
// residual |w| - mid q decides: one fused multiply-add rounds it once, and a
// nonzero residual cannot round to zero here (both terms are multiples of
// 2^-149 when q >= 2^-96), so the sign is exact; zero is a tie, resolved to
// the even neighbour (the parity of the lower end's three bits).  If t sits a
// rounding away from an E4M3 value, the gap picked may be the one on the
// other side of that value; the midpoint test then still returns the value
// itself.  The code of the lower end is its float32 bits >> 20 (exponent
// and the three bits) less the exponent bias difference; a carry into the
// next binade gives the next code, as E4M3 codes run in value order; the
// result is capped at 0x7E (448) as the float64 form does.
__device__ __forceinline__ uint32_t e4m3_code_rne_q(float w, float q, float rq) {
  const uint32_t sign = (__float_as_uint(w) >> 24) & 0x80u;
  const float a = fabsf(w);
  if (a != a) return sign | 0x7Fu;
  const float t = a * rq;
  if (!(t < 512.0f)) return sign | 0x7Eu;  // the quotient is far past 464
  const bool sub = t < 0x1p-6f;
  const float u = sub ? t + 0x1p-6f : t;
  const uint32_t b = __float_as_uint(u);
  const float mid_u = __uint_as_float((b & 0xFFF00000u) | 0x00080000u);
  const float mid = sub ? mid_u - 0x1p-6f : mid_u;
  const float d = fmaf(-mid, q, a);
  const int up = (d > 0.0f || (d == 0.0f && ((b >> 20) & 1u))) ? 1 : 0;
  const int code = (int)(b >> 20) - ((127 - 7) << 3) - (sub ? 8 : 0) + up;
  return sign | (uint32_t)min(code, 0x7E);
}

// One workgroup of kRowThreads per row (a weight's output channel, or a
// row of x): amax (exact), q = float32(float64(amax) / 448) (1 for a zero
// row), codes of |w| / q rounded to nearest even (float32 with an exact
// residual test; rows with q < 2^-96 take the float64 division).  Thread i
// holds the 16-byte pieces i, i + kRowThreads, ... of the row (8 bf16 or 4
// float32 values each), its first kKeep pieces in registers across the two
// passes (the whole row up to K = 4096 bf16 / 2048 float32 values; longer
// rows read the rest again).  A probe of four layouts on 4096 rows of 4096
// bf16 values measured this one fastest (18.0 us against 19.1-22.8 for one
// or two waves per row, a read-only pass taking 7.2): the rounding's
// arithmetic, not the memory, is most of the time, and it spreads best over
// 256 threads per row.  K is a multiple of 16, so every piece is whole and
// 16-byte aligned.
// STATS (rows of x for the fp8 prefill product): the same first read also
// sums the squares, and the row's factor s q with s = 1 / sqrt(mean(x^2) +
// eps) goes out in place of q (the deferred row scale, FlashNorm Abstract
// point (ii), multiplied into the dequantisation scale).
template <int WDT, bool STATS = false>
__global__ __launch_bounds__(kRowThreads) void quantize_fp8_kernel(const void* __restrict__ W, int64_t rows, int K,
                                                                  uint8_t* __restrict__ codes,
                                                                  float* __restrict__ q_out, float eps) {
  constexpr int PV = WDT == 0 ? 4 : 8;  // values per 16-byte piece
  constexpr int kKeep = 2;
  __shared__ float red[kRowThreads / 64];
  __shared__ float red_ss[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const int np = K / PV;  // pieces per row
  const u32x4* const src =
      reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(W) + row * (int64_t)K * (WDT == 0 ? 4 : 2));
  auto vals = [&](const u32x4& u, float v[PV]) {
    if constexpr (WDT == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(u[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(u[i]);
        v[2 * i + 1] = bf16_hi(u[i]);
      }
    }
  };
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 keep[kKeep];
#pragma unroll
  for (int u = 0; u < kKeep; ++u) {  // every kept piece is requested before the first is used
    const int c = threadIdx.x + kRowThreads * u;
    keep[u] = c < np ? src[c] : zero;
  }
  float amax = 0.f, ss = 0.f;
  auto take = [&](const u32x4& u) {
    float v[PV];
    vals(u, v);
#pragma unroll
    for (int i = 0; i < PV; ++i) {
      amax = fmaxf(amax, fabsf(v[i]));
      if constexpr (STATS) ss = fmaf(v[i], v[i], ss);
    }
  };
#pragma unroll
  for (int u = 0; u < kKeep; ++u) take(keep[u]);  // zero pieces change neither amax nor the sum
  for (int c = threadIdx.x + kRowThreads * kKeep; c < np; c += kRowThreads) take(src[c]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  if constexpr (STATS) ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = amax;
    red_ss[threadIdx.x >> 6] = ss;
  }
  __syncthreads();
  amax = 0.f;
  ss = 0.f;
#pragma unroll
  for (int i = 0; i < kRowThreads / 64; ++i) {
    amax = fmaxf(amax, red[i]);
    ss += red_ss[i];
  }
  const float q = amax > 0.f ? (float)((double)amax / 448.0) : 1.0f;
  if (threadIdx.x == 0) q_out[row] = STATS ? rsqrtf(ss * (1.0f / (float)K) + eps) * q : q;
  uint8_t* const dst = codes + row * (int64_t)K;
  const bool fast = q >= 0x1p-96f;  // row-uniform
  const float rq = 1.0f / q;
  const double qd = (double)q;
  // the PV codes of a piece, packed little-endian (the code of value i in byte i)
  auto put = [&](int c, const u32x4& u) {
    float v[PV];
    vals(u, v);
    uint32_t w[PV / 4];
#pragma unroll
    for (int h = 0; h < PV / 4; ++h) w[h] = 0;
    if (fast) {
#pragma unroll
      for (int i = 0; i < PV; ++i) w[i / 4] |= e4m3_code_rne_q(v[i], q, rq) << (8 * (i % 4));
    } else {
#pragma unroll
      for (int i = 0; i < PV; ++i) w[i / 4] |= e4m3_code_rne((double)v[i] / qd) << (8 * (i % 4));
    }
    if constexpr (PV == 8)
      *reinterpret_cast<uint2*>(dst + (int64_t)c * PV) = make_uint2(w[0], w[1]);
    else
      *reinterpret_cast<uint32_t*>(dst + (int64_t)c * PV) = w[0];
  };
#pragma unroll
  for (int u = 0; u < kKeep; ++u) {
    const int c = threadIdx.x + kRowThreads * u;
    if (c < np) put(c, keep[u]);
  }
  for (int c = threadIdx.x + kRowThreads * kKeep; c < np; c += kRowThreads) put(c, src[c]);
}

// MLA latent norms, one wave per row: for the q latent [0, nq) and the kv
// latent [nq, lat), the row's sum of squares from the GEMM's 32-column
// partial sums, then z * g / sqrt(mean + eps) in four-column pieces.
template <int ODT>
__global__ __launch_bounds__(kRowsPerBlock * 64) void latent_norm_kernel(const float* __restrict__ z,
                                                                         const float* __restrict__ part, int64_t M,
                                                                         int lat, int nq, const float* __restrict__ g_q,
                                                                         const float* __restrict__ g_kv, float eps,
                                                                         void* __restrict__ y, int64_t N) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* zr = z + row * lat;
  const float* pr = part + row * (lat / 32);
#pragma unroll
  for (int seg = 0; seg < 2; ++seg) {
    const int lo = seg ? nq : 0;
    const int w = seg ? lat - nq : nq;
    if (w == 0) continue;
    const float* g = seg ? g_kv : g_q;
    float t = 0.f;
    for (int q = lane; q < w / 32; q += 64) t += pr[lo / 32 + q];
    t = wave_sum(t);
    const float r = rsqrtf(t / (float)w + eps);
    for (int c = 4 * lane; c < w; c += 256) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(zr + lo + c);
      const f32x4 gg = *reinterpret_cast<const f32x4*>(g + c);
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = v[e] * r * gg[e];
      const int64_t off = row * N + lo + c;
      if constexpr (ODT == 0) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(y) + off) = f32x4{o[0], o[1], o[2], o[3]};
      } else {
        uint2 u;
        u.x = pack_bf16x2(o[0], o[1]);
        u.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + off) = u;
      }
    }
  }
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
  return launch_rows<ROW_RMSNORM>(x, dt, M, K, eps, g, nullptr, nullptr, nullptr, xn, st);
}

hipError_t launch_layernorm(const void* x, int dt, const float* g, const float* beta, int64_t M, int64_t K, float eps,
                            void* xn, hipStream_t st) {
  return launch_rows<ROW_LAYERNORM>(x, dt, M, K, eps, g, beta, nullptr, nullptr, xn, st);
}

hipError_t launch_fold_layernorm(const void* W, int w_dt, const float* g, const float* beta, const float* bias,
                                 int64_t N, int64_t K, void* Ws, int out_dt, float* c, float* b, hipStream_t st) {
  const dim3 grid((unsigned)N), block(kRowThreads);
  const int k = (int)K;
  if (w_dt == 0 && out_dt == 0)
    hipLaunchKernelGGL((fold_layernorm_kernel<0, 0>), grid, block, 0, st, W, g, beta, bias, k, Ws, c, b);
  else if (w_dt == 0 && out_dt == 1)
    hipLaunchKernelGGL((fold_layernorm_kernel<0, 1>), grid, block, 0, st, W, g, beta, bias, k, Ws, c, b);
  else if (w_dt == 1 && out_dt == 0)
    hipLaunchKernelGGL((fold_layernorm_kernel<1, 0>), grid, block, 0, st, W, g, beta, bias, k, Ws, c, b);
  else
    hipLaunchKernelGGL((fold_layernorm_kernel<1, 1>), grid, block, 0, st, W, g, beta, bias, k, Ws, c, b);
  return hipGetLastError();
}

hipError_t launch_ln_stats(const void* x, int dt, int64_t M, int64_t K, float eps, float* mu, float* s,
                           hipStream_t st) {
  return launch_rows<ROW_LN_STATS>(x, dt, M, K, eps, nullptr, nullptr, s, mu, nullptr, st);
}

hipError_t launch_row_scale(const void* x, int dt, int64_t M, int64_t K, float eps, float* s, hipStream_t st) {
  return launch_rows<ROW_SCALE>(x, dt, M, K, eps, nullptr, nullptr, s, nullptr, nullptr, st);
}

hipError_t launch_post_scale(const float* z, const float* s, int64_t M, int64_t N, void* y, int y_dt,
                             hipStream_t st) {
  const int64_t groups = M * N / 4;
  const int grid = grid_for(groups, 256);
  if (y_dt == 0) hipLaunchKernelGGL((post_scale_kernel<0>), dim3(grid), dim3(256), 0, st, z, s, groups, (int)N, y);
  else hipLaunchKernelGGL((post_scale_kernel<1>), dim3(grid), dim3(256), 0, st, z, s, groups, (int)N, y);
  return hipGetLastError();
}


hipError_t launch_quantize_fp8(const void* W, int w_dt, int64_t N, int64_t K, uint8_t* codes, float* q,
                               hipStream_t st) {
  const dim3 grid((unsigned)N), block(kRowThreads);
  if (w_dt == 0)
    hipLaunchKernelGGL((quantize_fp8_kernel<0>), grid, block, 0, st, W, N, (int)K, codes, q, 0.f);
  else
    hipLaunchKernelGGL((quantize_fp8_kernel<1>), grid, block, 0, st, W, N, (int)K, codes, q, 0.f);
  return hipGetLastError();
}

hipError_t launch_quantize_rows_fp8(const void* x, int64_t M, int64_t K, bool stats, float eps, uint8_t* codes,
                                    float* r, hipStream_t st) {
  const dim3 grid((unsigned)M), block(kRowThreads);
  if (stats)
    hipLaunchKernelGGL((quantize_fp8_kernel<1, true>), grid, block, 0, st, x, M, (int)K, codes, r, eps);
  else
    hipLaunchKernelGGL((quantize_fp8_kernel<1, false>), grid, block, 0, st, x, M, (int)K, codes, r, eps);
  return hipGetLastError();
}

hipError_t launch_latent_norm(const float* z, const float* part, int64_t M, int lat, int nq, const float* g_q,
                              const float* g_kv, float eps, void* y, int64_t N, int y_dt, hipStream_t st) {
  const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * 64);
  if (y_dt == 0)
    hipLaunchKernelGGL((latent_norm_kernel<0>), grid, block, 0, st, z, part, M, lat, nq, g_q, g_kv, eps, y, N);
  else
    hipLaunchKernelGGL((latent_norm_kernel<1>), grid, block, 0, st, z, part, M, lat, nq, g_q, g_kv, eps, y, N);
  return hipGetLastError();
}

namespace {

// One wave per (row, head) of the head-norm ops' decode path, four heads of
// a row per workgroup (single-wave workgroups measured 0.8 us per row
// slower, the dispatch of many tiny workgroups dominating).  A lane holds
// cpl consecutive columns of the head (4 for heads of 256, else 2; a head
// of 64 uses 32 lanes), so rotary pairs never straddle lanes.  Every load
// that does not depend on another is issued first (the product, the gains,
// the position, the row of x), so a wave waits for about two memory round
// trips in all.
template <int ODT, bool ROPE>
__global__ __launch_bounds__(256) void qk_finish_kernel(QkFinishArgs a) {
  // four heads of one row per workgroup, one wave each
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.y;
  const int head = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int hd = a.head_dim;
  if (head * hd >= a.N) return;  // wave-uniform: the last workgroup of a row may hold fewer heads
  const int c0 = head * hd;
  const bool is_q = c0 < a.nq_cols;
  const bool is_v = c0 >= a.nq_cols + a.nk_cols;
  const int cpl = hd >= 256 ? 4 : 2;
  const bool on = lane * cpl < hd;
  const int cih = lane * cpl;  // first column of the lane within the head
  const bool row_scale = is_v && a.v_mode == 0 && a.v_scale;
  // ---- loads ----
  int p = 0;
  if constexpr (ROPE) {
    if (!is_v) p = a.pos[m];
  }
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  float g[4] = {1.f, 1.f, 1.f, 1.f};
  if (on) {
    const float* zr = a.z + (size_t)m * a.N + c0 + cih;
    for (int r = 0; r < cpl; ++r) v[r] = zr[r];
    if (!is_v) {
      const int nq_heads = a.nq_cols / hd;
      const float* gp = is_q ? a.g_q + (size_t)head * a.g_stride : a.g_k + (size_t)(head - nq_heads) * a.g_stride;
      for (int r = 0; r < cpl; ++r) g[r] = gp[cih + r];
    }
  }
  // the deferred row scale s[m] = 1 / sqrt(mean_k x[m,k]^2 + eps_x): four
  // independent 16-byte loads per lane in flight at a time
  float t4[4] = {0.f, 0.f, 0.f, 0.f};
  if (row_scale) {
    const uint16_t* xr = a.x + (size_t)m * a.K;
    int k = lane * 8;
    for (; k + 3 * 512 < a.K; k += 4 * 512) {
      u32x4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = *reinterpret_cast<const u32x4*>(xr + k + u * 512);
#pragma unroll
      for (int u = 0; u < 4; ++u) t4[u] = sumsq_bf16x8_dot2(q[u], t4[u]);
    }
    for (; k < a.K; k += 512) t4[0] = sumsq_bf16x8_dot2(*reinterpret_cast<const u32x4*>(xr + k), t4[0]);
  }
  // rotary (cos, sin) of the lane's pairs: pair i of the head is columns
  // 2i, 2i + 1, its values at t[pos * rot_dim + 2i .. + 1]
  float cs[4] = {1.f, 0.f, 1.f, 0.f};
  bool pos_ok = true;
  if constexpr (ROPE) {
    if (!is_v && on) {
      pos_ok = p >= 0 && p < a.n_pos;
      const float* trow = a.rope + (size_t)(pos_ok ? p : 0) * a.rot_dim;
      for (int r = 0; r < cpl; r += 2)
        if (cih + r < a.rot_dim) {
          cs[r] = trow[cih + r];
          cs[r + 1] = trow[cih + r + 1];
        }
    }
  }
  // ---- arithmetic ----
  float scale = 1.f;
  if (!is_v || a.v_mode == 1) {
    float ss = 0.f;
    for (int r = 0; r < cpl; ++r) ss = fmaf(v[r], v[r], ss);
    ss = wave_sum(ss);
    scale = rsqrtf(ss / (float)hd + a.eps_head);
  } else if (row_scale) {
    const float t = wave_sum((t4[0] + t4[1]) + (t4[2] + t4[3]));
    scale = rsqrtf(t * a.inv_k + a.eps_x);
  }
  for (int r = 0; r < 4; ++r) v[r] = v[r] * scale * g[r];
  if constexpr (ROPE) {
    // columns past rot_dim and v heads keep their values; a position
    // outside the table gives NaN
    if (!is_v) {
      const float qnan = __builtin_nanf("");
      for (int r = 0; r < cpl; r += 2)
        if (cih + r < a.rot_dim) {
          const float c = pos_ok ? cs[r] : qnan, sn = pos_ok ? cs[r + 1] : qnan;
          const float x0 = v[r], x1 = v[r + 1];
          v[r] = x0 * c - x1 * sn;
          v[r + 1] = x0 * sn + x1 * c;
        }
    }
  }
  if (on) {
    const size_t o = (size_t)m * a.N + c0 + cih;
    for (int r = 0; r < cpl; ++r) {
      if constexpr (ODT == 1)
        static_cast<uint16_t*>(a.y)[o + r] = out_bf16_bits(v[r]);
      else
        static_cast<float*>(a.y)[o + r] = v[r];
    }
  }
}

}  // namespace

hipError_t launch_qk_finish(const QkFinishArgs& a, int y_dt, hipStream_t st) {
  const dim3 grid((unsigned)((a.N / a.head_dim + 3) / 4), (unsigned)a.M), block(256);
  const bool rope = a.pos != nullptr;
  if (y_dt == 1) {
    if (rope) hipLaunchKernelGGL((qk_finish_kernel<1, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((qk_finish_kernel<1, false>), grid, block, 0, st, a);
  } else {
    if (rope) hipLaunchKernelGGL((qk_finish_kernel<0, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((qk_finish_kernel<0, false>), grid, block, 0, st, a);
  }
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
