// Decode kernel (M <= 16 rows): the product is bound by streaming W* from
// HBM, so the whole chip reads W* once, in wide loads, while x (a few KB)
// stays in cache.  v_mfma_f32_16x16x32_bf16 does the contraction with x as
// the 16-row A operand (rows >= M are zero) and 16 weight rows as B; the
// row sum of squares comes from the same x fragments (FlashNorm Abstract,
// point (ii): the scalar is applied to the product's output).
//
// Workgroup: 8 waves on one 32-row slab of W* (plain: 32 output columns;
// glu: 16 gate rows + the matching 16 up rows).  K is cut into 32-wide
// steps; a pass of the K loop gives each wave kUnroll steps, either
// consecutive (CONSEC: 256 contiguous bytes of each row per wave) or dealt
// round-robin.  Workgroups start their passes at different points of K so
// that, at any moment, the chip's reads spread over all of each row and so
// over the memory channels.  Partial accumulators and sums of squares are
// combined through LDS, then one wave applies the epilogue.  The LayerNorm
// epilogue also takes the row mean from shifted sums of x kept alongside
// the squares, and subtracts mean * (column sum of W*) before the scale.
//
// Weights are read either row-major (16 rows x 64 bytes per load
// instruction of a wave) or in the decode-packed layout (PK), in which each
// 16-row slab stores every 64-byte K step as the 64 lane pieces of one
// wave load, back to back: a load then covers 1 KB of contiguous memory and
// a workgroup walks its slabs front to back.  For the glu epilogue the gate
// and up weights can share one buffer (PAIR): each 2 KB K step holds the
// gate slab's pieces, then the up slab's, so a workgroup's reads form one
// contiguous run.  Every layout reads the same values into the same lanes,
// so the arithmetic is the same.  fp8 weights (F8) use the same layouts
// with 64-value steps.

#include <cstdlib>
#include <cstring>

#include "common.hpp"
#include "kernels.hpp"

namespace fn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kUnroll = 4;

constexpr int kXLdsElems = 16384;  // x rows staged in LDS when M * K fits (32 KB)

// E4M3 weights (F8): 16 bytes of a weight row per lane and step, widened
// in registers to bf16 (exact: an E4M3 value has at most 4 significant
// bits) by the hardware's scaled conversion with scale 1, two codes per
// instruction, code 2i to the low half of word i; then the same bf16 MFMAs.
// Checked against the float32 conversion for all 256 codes in every byte
// position: identical bits.
__device__ __forceinline__ void dequant_e4m3x16(const u32x4& w, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
    const uint32_t d1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    if (i < 2) {
      lo[2 * i] = d0;
      lo[2 * i + 1] = d1;
    } else {
      hi[2 * i - 4] = d0;
      hi[2 * i - 3] = d1;
    }
  }
}

template <int EPI, bool SUMSQ, bool OUT_BF16, bool CONSEC, int NB, bool XL, bool F8 = false, bool PK = false,
          bool PAIR = false>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(DecodeArgs p) {
  static_assert(NB == 2 || NB == 4 || (NB == 1 && EPI == EPI_PLAIN), "1 (plain), 2 or 4 16-row weight slabs");
  constexpr int HB = NB >= 2 ? NB / 2 : 1;  // glu: gate slabs per workgroup
  static_assert(!F8 || EPI != EPI_LN, "fp8 weights: plain or glu epilogue");
  // K step of one MFMA pass: 32 (bf16 weights, 8 per lane) or 64 (fp8
  // weights, 16 per lane, two MFMAs: the same k permutation on x and W*)
  constexpr int KSTEP = F8 ? 64 : 32;
  constexpr int XH = F8 ? 2 : 1;  // 16-byte x pieces per lane and step
  constexpr int WB = F8 ? 1 : 2;  // weight bytes per element
  // Steps per wave and pass.  fp8: three, which keeps the kernel at <= 80
  // VGPRs, so three workgroups fit per CU and the Llama-7B FFN grid (688
  // workgroups) runs in one round; four steps take 93 VGPRs and two rounds.
  constexpr int KU = F8 ? 3 : kUnroll;
  constexpr bool LNS = (EPI == EPI_LN) && SUMSQ;  // LayerNorm statistics
  __shared__ f32x4 red_acc[kWaves][NB][64];
  __shared__ float red_ss[kWaves][64];
  __shared__ float red_s1[LNS ? kWaves : 1][64];
  // XL: the M x K rows of x are copied to LDS once, so the K loop issues
  // only weight loads to memory (the launcher picks XL when M K fits).
  __shared__ __attribute__((aligned(16))) uint16_t xs[XL ? kXLdsElems : 8];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int frow = lane & 15;
  const int fchk = lane >> 4;
  const int M = p.M, K = p.K, N = p.N;

  // The NB 16-row B slabs of this workgroup.  glu: the first NB/2 are gate
  // rows, the rest the matching up rows; plain: NB consecutive slabs.
  constexpr int OUT_COLS = (EPI == EPI_GLU) ? 16 * NB / 2 : 16 * NB;
  const int n_out0 = blockIdx.x * OUT_COLS;  // first output column
  const uint8_t* bp[NB];  // weight rows (PK: this lane's piece of the slab's first step), as bytes
  // PAIR (glu): gate and up packed into one buffer, each K step of slab j
  // holding the gate piece then the up piece (2 KB).
  static_assert(!PAIR || (PK && EPI == EPI_GLU), "the gate/up pair layout is a packed glu layout");
  constexpr int SSTEP = PAIR ? 2048 : 1024;  // bytes from one K step of a slab to the next
  if constexpr (PK) {
    const int slabs = (N + 15) / 16;
    const size_t slab_bytes = (size_t)((K + KSTEP - 1) / KSTEP) * SSTEP;
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      const int j = min((n_out0 + 16 * ((EPI == EPI_GLU) ? s % HB : s)) / 16, slabs - 1);
      const bool up = EPI == EPI_GLU && s >= NB / 2;
      const void* base = (up && !PAIR) ? p.B1 : p.B0;
      bp[s] = reinterpret_cast<const uint8_t*>(base) + (size_t)j * slab_bytes + ((PAIR && up) ? 1024 : 0) + lane * 16;
    }
  } else {
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    if constexpr (EPI == EPI_GLU) {
      const int n = min(n_out0 + 16 * (s % (NB / 2)) + frow, N - 1);
      bp[s] = reinterpret_cast<const uint8_t*>(s < NB / 2 ? p.B0 : p.B1) + (size_t)n * K * WB;
    } else {
      bp[s] = reinterpret_cast<const uint8_t*>(p.B0) + (size_t)min(n_out0 + 16 * s + frow, N - 1) * K * WB;
    }
  }
  }
  const bool row_ok = frow < M;
  const uint16_t* xa = p.x + (size_t)(row_ok ? frow : 0) * K;
  const uint16_t* xl = xs + (row_ok ? frow : 0) * K;

  f32x4 acc[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  // LayerNorm: sums of x - sh and (x - sh)^2, sh = the row's first element
  float s1 = 0.f;
  const int steps = (K + KSTEP - 1) / KSTEP;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int passes = (steps + kWaves * KU - 1) / (kWaves * KU);

  // K step of the lane's piece u in pass it, and the pass's weight pieces
  auto step_of = [&](int it, int u) {
    return CONSEC ? (it * kWaves + wave) * KU + u : it * kWaves * KU + wave + u * kWaves;
  };
  auto load_w = [&](int it, u32x4 (&w)[KU][NB]) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int st = step_of(it, u);
      const int k = st * KSTEP + fchk * 8 * XH;  // K % (8 XH) == 0: whole pieces
      const bool ok = (st < steps) && (k < K);
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        const uint8_t* wp = PK ? bp[s] + (size_t)st * SSTEP : bp[s] + (size_t)k * WB;
        w[u][s] = ok ? *reinterpret_cast<const u32x4*>(wp) : zero;
      }
    }
  };
  // The lane's x pieces of a pass (from LDS or memory); with `w` non-null the
  // weight pieces of each step are requested right after that step's x
  // pieces (the order the memory-resident x needs: a step's MFMAs wait only
  // for the loads issued before its own).
  float sh = 0.f;
  auto load_x = [&](int it, u32x4 (&a)[KU][XH], bool (&aok)[KU], u32x4 (*w)[NB]) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int st = step_of(it, u);
      const int k = st * KSTEP + fchk * 8 * XH;
      const bool ok = (st < steps) && (k < K);
      aok[u] = ok && row_ok;
#pragma unroll
      for (int h = 0; h < XH; ++h) {
        if constexpr (XL)
          a[u][h] = (ok && row_ok) ? *reinterpret_cast<const u32x4*>(xl + k + 8 * h) : zero;
        else
          a[u][h] = (ok && row_ok) ? *reinterpret_cast<const u32x4*>(xa + k + 8 * h) : zero;
      }
      if (w != nullptr) {
#pragma unroll
        for (int s = 0; s < NB; ++s) {
          const uint8_t* wp = PK ? bp[s] + (size_t)st * SSTEP : bp[s] + (size_t)k * WB;
          w[u][s] = ok ? *reinterpret_cast<const u32x4*>(wp) : zero;
        }
      }
    }
  };
  // The squares of a pass's x pieces and its MFMAs.
  auto compute = [&](const u32x4 (&a)[KU][XH], const bool (&aok)[KU], const u32x4 (&w)[KU][NB]) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
#pragma unroll
      for (int h = 0; h < XH; ++h) {
        if constexpr (LNS) {
          if (aok[u]) lnstat_bf16x8(a[u][h], sh, s1, ss);  // chunks past K (zeros) must not count
        } else if constexpr (SUMSQ) {
          ss = sumsq_bf16x8_dot2(a[u][h], ss);
        }
      }
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        if constexpr (F8) {
          u32x4 lo, hi;
          dequant_e4m3x16(w[u][s], lo, hi);
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u][0]),
                                                           __builtin_bit_cast(bf16x8, lo), acc[s], 0, 0, 0);
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u][1]),
                                                           __builtin_bit_cast(bf16x8, hi), acc[s], 0, 0, 0);
        } else {
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[u][0]),
                                                           __builtin_bit_cast(bf16x8, w[u][s]), acc[s], 0, 0, 0);
        }
      }
    }
  };

  // Passes start at staggered points of K (pass it = (it0 + workgroup) %
  // passes).
  if constexpr (XL) {
    // The first pass's weights are requested before anything else, ahead of
    // the x copy into LDS and its barrier, so the workgroup's weight stream
    // starts with the workgroup (6-7% at M = 4, 3% at M = 1).
    const int it_first = (int)(blockIdx.x % (unsigned)passes);
    u32x4 w[KU][NB];
    load_w(it_first, w);
    const int chunks = M * K / 8;  // K % 8 == 0
    for (int c = threadIdx.x; c < chunks; c += kThreads)
      *reinterpret_cast<u32x4*>(xs + c * 8) = *reinterpret_cast<const u32x4*>(p.x + (size_t)c * 8);
    __syncthreads();
    if constexpr (LNS) sh = row_ok ? __uint_as_float((uint32_t)xa[0] << 16) : 0.f;
    u32x4 a[KU][XH];
    bool aok[KU];
    load_x(it_first, a, aok, nullptr);
    compute(a, aok, w);
    for (int it0 = 1; it0 < passes; ++it0) {
      const int it = (it0 + (int)blockIdx.x) % passes;
      load_w(it, w);
      load_x(it, a, aok, nullptr);
      compute(a, aok, w);
    }
  } else {
    if constexpr (LNS) sh = row_ok ? __uint_as_float((uint32_t)xa[0] << 16) : 0.f;
    for (int it0 = 0; it0 < passes; ++it0) {
      const int it = (it0 + (int)blockIdx.x) % passes;
      u32x4 a[KU][XH], w[KU][NB];
      bool aok[KU];
      load_x(it, a, aok, w);
      compute(a, aok, w);
    }
  }
#pragma unroll
  for (int s = 0; s < NB; ++s) red_acc[wave][s][lane] = acc[s];
  red_ss[wave][lane] = ss;
  if constexpr (LNS) red_s1[wave][lane] = s1;
  __syncthreads();
  if (wave != 0) return;

  f32x4 c[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) c[s] = red_acc[0][s][lane];
  float t = red_ss[0][lane];
  float t1 = LNS ? red_s1[0][lane] : 0.f;
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
#pragma unroll
    for (int s = 0; s < NB; ++s) c[s] += red_acc[w][s][lane];
    t += red_ss[w][lane];
    if constexpr (LNS) t1 += red_s1[w][lane];
  }
  // accumulator lane layout: row 4 * (lane / 16) + r, column lane % 16
  float srow[4], mrow[4];
  if constexpr (LNS) {
    t = xor_sum<32>(xor_sum<16>(t));
    t1 = xor_sum<32>(xor_sum<16>(t1));
    const float md = t1 * p.inv_k;  // lane j (< 16) holds row j's sums and shift
    const float sc = rsqrtf(fmaxf(fmaf(-md, md, t * p.inv_k), 0.f) + p.eps);
    const float mu = sh + md;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      srow[r] = __shfl(sc, 4 * fchk + r, kWave);
      mrow[r] = __shfl(mu, 4 * fchk + r, kWave);
    }
  } else if constexpr (SUMSQ) {
    t = xor_sum<16>(t);
    t = xor_sum<32>(t);
    const float sc = rsqrtf(t * p.inv_k + p.eps);  // lane j (< 16) holds row j's scale
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      srow[r] = __shfl(sc, 4 * fchk + r, kWave);
      mrow[r] = 0.f;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      srow[r] = 1.0f;
      mrow[r] = 0.f;
    }
  }

  auto store = [&](int m, int n, float v) {
    if (m < M && n < N) {
      if constexpr (OUT_BF16)
        static_cast<uint16_t*>(p.Y)[(size_t)m * N + n] = out_bf16_bits(v);
      else
        static_cast<float*>(p.Y)[(size_t)m * N + n] = v;
    }
  };
  // fp8: the channel scales of this lane's columns
  float qg[NB], qu[NB];
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    qg[s] = qu[s] = 1.f;
    if constexpr (F8) {
      const int n = min(n_out0 + 16 * (EPI == EPI_GLU ? s % HB : s) + frow, N - 1);
      qg[s] = p.q0[n];
      if constexpr (EPI == EPI_GLU) qu[s] = p.q1[n];
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * fchk + r;
    if constexpr (EPI == EPI_GLU) {
#pragma unroll
      for (int s = 0; s < NB / 2; ++s) {
        const float a = F8 ? c[s][r] * srow[r] * qg[s] : c[s][r] * srow[r];
        const float b = F8 ? c[s + NB / 2][r] * srow[r] * qu[s] : c[s + NB / 2][r] * srow[r];
        store(m, n_out0 + 16 * s + frow, silu(a) * b);
      }
    } else if constexpr (EPI == EPI_LN) {
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        const int n = n_out0 + 16 * s + frow;
        const float cn = (LNS && n < N) ? p.ln_c[n] : 0.f;
        const float bn = (p.ln_b != nullptr && n < N) ? p.ln_b[n] : 0.f;
        store(m, n, fmaf(fmaf(-mrow[r], cn, c[s][r]), srow[r], bn));
      }
    } else {
#pragma unroll
      for (int s = 0; s < NB; ++s)
        store(m, n_out0 + 16 * s + frow, F8 ? c[s][r] * srow[r] * qg[s] : c[s][r] * srow[r]);
    }
  }
}

// One thread per 16-byte piece of the decode-packed layout: piece p of
// step st of slab j holds row 16 j + p % 16, bytes 64 st + 16 (p / 16) ..
// + 15 of that row; rows >= N and bytes >= the row's length are zero.
// With W1 (the gate/up pair layout) each step holds W0's 64 pieces, then
// W1's.
__global__ __launch_bounds__(256) void pack_decode_kernel(const uint8_t* __restrict__ W0,
                                                          const uint8_t* __restrict__ W1, int64_t N,
                                                          int64_t row_bytes, int64_t steps, int64_t pieces,
                                                          uint8_t* __restrict__ P) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= pieces) return;
  const int pc = (int)(q & 63);
  int64_t t = q >> 6;
  const uint8_t* W = W0;
  if (W1 != nullptr) {
    W = (t & 1) ? W1 : W0;
    t >>= 1;
  }
  const int64_t st = t % steps;
  const int64_t row = 16 * (t / steps) + (pc & 15);
  const int64_t kb = 64 * st + 16 * (pc >> 4);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < N && kb < row_bytes) v = *reinterpret_cast<const u32x4*>(W + row * row_bytes + kb);
  *reinterpret_cast<u32x4*>(P + q * 16) = v;
}

// FN_DECODE_ORDER=consec / rr forces the bf16 kernel's step order (a
// tuning aid); -1 when unset or unknown.
int decode_order_override() {
  const char* v = std::getenv("FN_DECODE_ORDER");
  if (!v) return -1;
  if (std::strcmp(v, "consec") == 0) return 1;
  if (std::strcmp(v, "rr") == 0) return 0;
  return -1;
}

}  // namespace

hipError_t launch_pack_decode(const void* W, const void* W_up, int64_t N, int64_t row_bytes, void* P,
                              hipStream_t st) {
  const int64_t steps = (row_bytes + 63) / 64;
  const int64_t pieces = (N + 15) / 16 * steps * 64 * (W_up != nullptr ? 2 : 1);
  if (pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_decode_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st,
                     static_cast<const uint8_t*>(W), static_cast<const uint8_t*>(W_up), N, row_bytes, steps, pieces,
                     static_cast<uint8_t*>(P));
  return hipGetLastError();
}

hipError_t launch_decode_fp8(int epi, bool sumsq, bool out_bf16, const DecodeArgs& a, hipStream_t st) {
  // Round-robin steps at every M (with fp8 steps, consecutive ones measured
  // 3-4% slower at M <= 4), x in LDS when it fits.
  constexpr int NB = 2;
  const bool xl = (int64_t)a.M * a.K <= kXLdsElems;
  const int cols = ((epi == EPI_GLU) ? 8 : 16) * NB;
  const int grid = (a.N + cols - 1) / cols;
#define FN_DEC8(E, S, O)                                                                                   \
  do {                                                                                                     \
    if constexpr (E == EPI_GLU) {                                                                          \
      if (a.packed == 2) {                                                                                 \
        if (xl)                                                                                            \
          hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, true, true, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
        else                                                                                               \
          hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, false, true, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
        break;                                                                                             \
      }                                                                                                    \
    }                                                                                                      \
    if (a.packed && xl)                                                                                    \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, true, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
    else if (a.packed)                                                                                     \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, false, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
    else if (xl)                                                                                           \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
    else                                                                                                   \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, false, true>), dim3(grid), dim3(kThreads), 0, st, a); \
  } while (0)
  if (epi == EPI_GLU) {
    if (sumsq) { if (out_bf16) FN_DEC8(EPI_GLU, true, true); else FN_DEC8(EPI_GLU, true, false); }
    else       { if (out_bf16) FN_DEC8(EPI_GLU, false, true); else FN_DEC8(EPI_GLU, false, false); }
  } else if (epi == EPI_PLAIN) {
    if (sumsq) { if (out_bf16) FN_DEC8(EPI_PLAIN, true, true); else FN_DEC8(EPI_PLAIN, true, false); }
    else       { if (out_bf16) FN_DEC8(EPI_PLAIN, false, true); else FN_DEC8(EPI_PLAIN, false, false); }
  } else {
    return hipErrorInvalidValue;
  }
#undef FN_DEC8
  return hipGetLastError();
}

hipError_t launch_decode_bf16(int epi, bool sumsq, bool out_bf16, const DecodeArgs& a, hipStream_t st) {
  // Two weight slabs per workgroup (four measured slower at every M: half
  // as many workgroups).  Row-major weights: consecutive steps per wave
  // read best for a few rows; with more rows the round-robin order measured
  // faster.  Packed weights, measured at M = 1, 4 and 16: round-robin for
  // the glu epilogue (gate and up, two streams; 2-3% faster), consecutive
  // steps for one weight (plain and LayerNorm epilogues; 2-4% faster).
  constexpr int NB = 2;
  const int order = decode_order_override();
  const bool consec = order >= 0 ? order == 1 : (a.packed ? epi != EPI_GLU : a.M <= 4);
  const bool xl = (int64_t)a.M * a.K <= kXLdsElems;
  if (epi == EPI_PLAIN && !sumsq && !out_bf16 && !a.packed && (a.N + 31) / 32 < 256) {
    // A narrow float32 product (the head-norm ops' decode path): one slab of
    // 16 columns per workgroup, so the grid still covers the CUs.
    const int grid1 = (a.N + 15) / 16;
    if (consec && xl)
      hipLaunchKernelGGL((decode_bf16_kernel<EPI_PLAIN, false, false, true, 1, true>), dim3(grid1), dim3(kThreads), 0,
                         st, a);
    else if (consec)
      hipLaunchKernelGGL((decode_bf16_kernel<EPI_PLAIN, false, false, true, 1, false>), dim3(grid1), dim3(kThreads),
                         0, st, a);
    else
      hipLaunchKernelGGL((decode_bf16_kernel<EPI_PLAIN, false, false, false, 1, false>), dim3(grid1),
                         dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  const int cols = ((epi == EPI_GLU) ? 8 : 16) * NB;
  const int grid = (a.N + cols - 1) / cols;
#define FN_DEC(E, S, O)                                                                                        \
  do {                                                                                                         \
    if constexpr (E == EPI_GLU) {                                                                              \
      if (a.packed == 2) {                                                                                     \
        if (consec && xl)                                                                                      \
          hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, true, NB, true, false, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
        else if (consec)                                                                                       \
          hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, true, NB, false, false, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
        else if (xl)                                                                                           \
          hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, true, false, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
        else                                                                                                   \
          hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, false, false, true, true>), dim3(grid), dim3(kThreads), 0, st, a); \
        break;                                                                                                 \
      }                                                                                                        \
    }                                                                                                          \
    if (a.packed && consec && xl)                                                                              \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, true, NB, true, false, true>), dim3(grid), dim3(kThreads), 0, st, a); \
    else if (a.packed && consec)                                                                               \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, true, NB, false, false, true>), dim3(grid), dim3(kThreads), 0, st, a); \
    else if (a.packed && xl)                                                                                   \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, true, false, true>), dim3(grid), dim3(kThreads), 0, st, a); \
    else if (a.packed)                                                                                         \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, false, false, true>), dim3(grid), dim3(kThreads), 0, st, a); \
    else if (consec && xl)                                                                                     \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, true, NB, true>), dim3(grid), dim3(kThreads), 0, st, a);  \
    else if (consec)                                                                                           \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, true, NB, false>), dim3(grid), dim3(kThreads), 0, st, a); \
    else                                                                                                       \
      hipLaunchKernelGGL((decode_bf16_kernel<E, S, O, false, NB, false>), dim3(grid), dim3(kThreads), 0, st, a); \
  } while (0)
  if (epi == EPI_GLU) {
    if (sumsq) { if (out_bf16) FN_DEC(EPI_GLU, true, true); else FN_DEC(EPI_GLU, true, false); }
    else       { if (out_bf16) FN_DEC(EPI_GLU, false, true); else FN_DEC(EPI_GLU, false, false); }
  } else if (epi == EPI_PLAIN) {
    if (sumsq) { if (out_bf16) FN_DEC(EPI_PLAIN, true, true); else FN_DEC(EPI_PLAIN, true, false); }
    else       { if (out_bf16) FN_DEC(EPI_PLAIN, false, true); else FN_DEC(EPI_PLAIN, false, false); }
  } else if (epi == EPI_LN) {
    if (sumsq) { if (out_bf16) FN_DEC(EPI_LN, true, true); else FN_DEC(EPI_LN, true, false); }
    else       { if (out_bf16) FN_DEC(EPI_LN, false, true); else FN_DEC(EPI_LN, false, false); }
  } else {
    return hipErrorInvalidValue;
  }
#undef FN_DEC
  return hipGetLastError();
}

}  // namespace fn
