// Prefill kernel: bf16 MFMA contraction with the row sum of squares taken
// from the same x tiles that feed the matrix cores, and the deferred row
// scale applied in the epilogue (FlashNorm Abstract, points (i) and (ii)).
//
//   z[m, n] = sum_k x[m, k] * W*[n, k]     x [M x K], W* [N x K], both
//                                           K-contiguous bf16; fp32 accumulate
//   ss[m]   = sum_k x[m, k]^2               VALU, from the staged x tiles
//   s[m]    = 1 / sqrt(ss[m] / K + eps)
//   epilogue: plain  y = z * s
//             glu    h = SiLU(s * z_gate) * (s * z_up)
//             qknorm per-head RMSNorm of z on q/k heads, v = z * s (or normed)
//             qknorm_rope  the same, then q/k heads turned by the rotary
//                    embedding of the row's position
//             latent MLA attention input: latent columns to a float32
//                    workspace with per-32-column sums of squares (a row
//                    kernel applies the latent norms), the rest z * s (and
//                    the rotary embedding)
//             ln     LayerNorm: y = s (z - mu c[n]) + b[n], with the row's
//                    mean mu and s = 1 / sqrt(var + eps) from shifted sums
//                    of x and x^2 taken alongside, c = column sums of W*
//
// Layout and pipeline (gfx950):
//  * Workgroup tile BM x BN, K step 64, 8 waves (WAVES_M x WAVES_N), two per
//    SIMD, so one wave's LDS, barrier and memory waits hide behind the other
//    wave's MFMAs.  Each wave owns a (BN/WAVES_N) x (BM/WAVES_M) block of
//    32x32 accumulators (v_mfma_f32_32x32x16_bf16) with W* as the A operand
//    and x as the B operand: the accumulator is z transposed, so a lane holds
//    one output row m (= lane % 32) and runs of 4 consecutive columns n.
//  * Operands stream HBM -> LDS with buffer_load_dwordx4 ... lds (no staging
//    registers): one load instruction fills 8 rows x 128 B of a stage.  A
//    stage keeps rows of 64 bf16 (128 B); the eight 16-byte chunks of row r
//    sit at slot (chunk ^ ((r / 2) % 8)), so the 16 consecutive rows a
//    fragment read touches per LDS cycle hit distinct banks; the loads pick
//    the global chunk per lane so the bytes land in that order.
//  * A ring of NS LDS stages (separate objects, so the compiler can tell a
//    fragment read of one stage from an in-flight load into another), one
//    barrier per K step.  A K step is four 16-wide sub-steps; the fragments
//    of sub-step s+1 are read into a second register set while the MFMAs of
//    sub-step s run.  Before the last sub-step's MFMAs each wave waits for
//    its own loads of the next tile, the barrier is taken, the next tile's
//    first fragments are read, and tile kt+NS is requested into the stage
//    just finished.  Large tiles use two stages; small tiles, with little
//    work per K step, a deeper ring.
//  * The squares are VALU work beside the MFMAs, in one of two ways: from
//    the x fragments (where two waves share the same x rows, each squares
//    half of them and the sums are swapped through LDS at the end), or in
//    one pass per K step over the stage's x tile, dealt evenly to all
//    threads (cheaper for tiles whose waves share x rows four ways).
//  * bf16 outputs of interior tiles go through LDS so that every global
//    store writes whole row segments; edge tiles store directly with masks.
//  * Buffer resources start at the tile's first row and end at the tensor's
//    last row, so rows past M or N read as zeros.  A ragged last K step
//    (K % 64 != 0) goes through registers with lane masks after the loop.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace fn {

namespace {

constexpr int BK = 64;

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte chunk c of row r lives in slot c ^ ((r / 2) % 8) of the row.  A
// row is 128 B, so two consecutive rows fill the 64 banks once; a fragment
// read covers 16 consecutive rows per LDS cycle, whose 8 even (and 8 odd)
// rows then use 8 distinct slots: no bank conflicts.
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3); }

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for the stage ring: this wave's fragment reads are
// complete, then every wave meets.  Unlike __syncthreads() it does not wait
// for all of the wave's loads into LDS (the ring keeps later stages in
// flight); the caller waits for the ones the next stage needs.  The asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector-memory instructions are in
// flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NS, int SQM, bool W3, int EPI, bool SUMSQ, bool OUT_BF16,
          bool F8 = false, bool X3 = false>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64, 1) void gemm_bf16_kernel(GemmArgs p) {
  // X3: the mirror of W3, a third stage for the x tile alone (x requested
  // two K steps ahead, the weight tile one).
  static_assert(!X3 || (NS == 2 && !W3 && EPI == EPI_PLAIN && !F8), "the extra x stage: plain two-stage tiles");
  // F8: both operands are E4M3 codes (x quantised per row by a pass before
  // the kernel, W* per output channel).  A stage row still holds 128 bytes,
  // now 128 values, and a K step is two sub-steps of the 32x32x64 fp8 MFMA;
  // the epilogue multiplies by the row factor (row scale times x's
  // quantisation scale) and the weight's channel scale.
  static_assert(!F8 || !SUMSQ, "fp8: the row statistics come from the quantisation pass");
  static_assert(!F8 || EPI == EPI_PLAIN || EPI == EPI_GLU, "fp8: plain or glu epilogue");
  constexpr int EB = F8 ? 1 : 2;        // bytes per element
  constexpr int BKE = F8 ? 128 : BK;    // elements per K step (128 bytes of a row either way)
  constexpr int NSUB = F8 ? 2 : 4;      // MFMA sub-steps per K step
  constexpr int FW = F8 ? 2 : 1;        // 16-byte pieces per lane and fragment
  constexpr int CE = 16 / EB;           // elements per 16-byte chunk
  // W3: with two stages, a third stage for the weight tile alone, so weight
  // tiles (the operand re-read from farther away) are requested two K steps
  // ahead while x tiles stay one step ahead.
  static_assert(!W3 || NS == 2, "the extra weight stage extends a two-stage ring");
  static_assert(NS >= 2 && NS <= 4, "two to four LDS stages");
  static_assert(SQM == 0 || SQM == 1, "squares from fragments (0) or from the LDS x tile (1)");
  constexpr int kWaves = WAVES_M * WAVES_N;
  constexpr int kThreads = kWaves * 64;
  static_assert(kWaves == 4 || kWaves == 8, "one or two waves per SIMD");
  constexpr int WTN = BN / WAVES_N;  // W* rows (output columns before gating) per wave
  constexpr int WTM = BM / WAVES_M;  // x rows per wave
  constexpr int TJ = WTN / 32;       // 32-row W* subtiles per wave
  constexpr int TI = WTM / 32;       // 32-row x subtiles per wave
  constexpr int X_GROUPS = BM / 8 / kWaves;  // 8-row load groups per wave
  constexpr int W_GROUPS = BN / 8 / kWaves;
  static_assert(X_GROUPS >= 1 && W_GROUPS >= 1 && TJ >= 1 && TI >= 1, "tile too small for 8 waves");
  static_assert(EPI != EPI_GLU || (TJ % 2) == 0, "glu pairs gate/up subtiles");
  constexpr int OUT_BN = (EPI == EPI_GLU) ? BN / 2 : BN;  // output columns per tile
  constexpr int WOUT = (EPI == EPI_GLU) ? WTN / 2 : WTN;  // output columns per wave

  // One object per stage: the compiler then knows which stage a fragment
  // read touches and waits only for loads into that stage.
  // x and W* tiles of a stage are separate objects too, so a load into one
  // never looks like it could alias a fragment read of the other.
  constexpr int XE = BM * BK, WE = BN * BK;  // elements per x / W* stage
  __shared__ __attribute__((aligned(16))) uint16_t sx0[XE];
  __shared__ __attribute__((aligned(16))) uint16_t sx1[XE];
  __shared__ __attribute__((aligned(16))) uint16_t sx2[(NS > 2 || X3) ? XE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sx3[NS > 3 ? XE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sw0[WE];
  __shared__ __attribute__((aligned(16))) uint16_t sw1[WE];
  __shared__ __attribute__((aligned(16))) uint16_t sw2[(NS > 2 || W3) ? WE : 8];
  __shared__ __attribute__((aligned(16))) uint16_t sw3[NS > 3 ? WE : 8];
  uint16_t* const sX0 = sx0;
  uint16_t* const sW0 = sw0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int wn = wave % WAVES_N;
  const int wm = wave / WAVES_N;

  // ---- tile coordinates (XCD-aware, grouped along M) --------------------
  const int nblk = p.tiles_m * p.tiles_n;
  const int lin = xcd_remap(blockIdx.x, nblk);
  const int group = p.group_m;
  const int in_group = group * p.tiles_n;
  const int gid = lin / in_group;
  const int first_m = gid * group;
  const int gsize = min(p.tiles_m - first_m, group);
  const int tile_m = first_m + (lin % in_group) % gsize;
  const int tile_n = (lin % in_group) / gsize;
  const int m0 = tile_m * BM;
  const int n0 = tile_n * OUT_BN;

  const int M = p.M, K = p.K, N = p.N;
  const int KT = K / BKE;  // full K steps
  const bool k_tail = (K % BKE) != 0;

  // ---- buffer resources ----------------------------------------------------
  auto make_rsrc = [&](const uint16_t* base, int rows_left) {
    const int64_t bytes = (int64_t)rows_left * K * EB;
    const int nrec = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nrec, 0x00020000);
  };
  auto rows_at = [&](const uint16_t* base, int row) {
    return reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(base) + (size_t)row * K * EB);
  };
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(rows_at(p.A, m0), M - m0);
  const __amdgpu_buffer_rsrc_t rs_w0 = make_rsrc(rows_at(p.B0, n0), N - n0);
  const __amdgpu_buffer_rsrc_t rs_w1 = (EPI == EPI_GLU) ? make_rsrc(rows_at(p.B1, n0), N - n0) : rs_w0;

  // Direct loads: lane l of 8-row group g fills LDS slot l % 8 of row
  // 8 g + l / 8, which holds global chunk (l % 8) ^ ((8 g + l / 8) / 2 % 8)
  // = (l % 8) ^ (4 (g % 2) + l / 16).
  const int g_row = lane >> 3;
  const int voff_even = g_row * K * EB + (((lane & 7) ^ (lane >> 4)) << 4);
  const int voff_odd = g_row * K * EB + (((lane & 7) ^ ((lane >> 4) | 4)) << 4);
  const int group_bytes = 8 * K * EB;

  auto issue_x = [&](uint16_t* sX, int kt) {
    const int kb = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < X_GROUPS; ++i) {
      const int g = wave * X_GROUPS + i;
      const int voff = (g & 1) ? voff_odd : voff_even;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_x, (lds_void*)(sX + g * 8 * BK), 16, voff, g * group_bytes + kb, 0,
                                               0);
    }
  };
  auto issue_w = [&](uint16_t* sW, int kt) {
    const int kb = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < W_GROUPS; ++i) {
      const int g = wave * W_GROUPS + i;
      const int voff = (g & 1) ? voff_odd : voff_even;
      if constexpr (EPI == EPI_GLU) {
        constexpr int HALF = BN / 16;  // groups of gate rows
        if (g < HALF)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w0, (lds_void*)(sW + g * 8 * BK), 16, voff,
                                                   g * group_bytes + kb, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w1, (lds_void*)(sW + g * 8 * BK), 16, voff,
                                                   (g - HALF) * group_bytes + kb, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w0, (lds_void*)(sW + g * 8 * BK), 16, voff, g * group_bytes + kb,
                                                 0, 0);
      }
    }
  };
  auto issue_tile = [&](uint16_t* sX, uint16_t* sW, int kt) {
    issue_x(sX, kt);
    issue_w(sW, kt);
  };

  // ---- fragments -------------------------------------------------------------
  // 32x32x16 operands: lane l holds row l % 32 of a subtile (W* row for the A
  // operand, x row for the B operand) and the 8-element K chunk l / 32 of a
  // 16-wide K sub-step.  A K step of 64 is four sub-steps, taken in halves.
  const int frow = lane & 31;
  const int fchk = lane >> 5;
  int w_off[TJ], x_off[TI];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    if constexpr (EPI == EPI_GLU)
      w_off[j] = (j < TJ / 2) ? wn * (WTN / 2) + j * 32 + frow : BN / 2 + wn * (WTN / 2) + (j - TJ / 2) * 32 + frow;
    else
      w_off[j] = wn * WTN + j * 32 + frow;
  }
  // When NSPLIT waves share the same x subtiles, wave wn squares only its
  // share, kept in the first fragment slots (the slot order does not matter
  // to the MFMAs); the waves swap sums in the epilogue.
  // Squares, mode 0: from the x fragments each wave feeds its MFMAs.  Mode 1
  // (SQL): one pass per K step over the stage's x tile, the BM x 64 block
  // dealt evenly to all threads, so no two waves square the same values.
  constexpr bool SQL = SUMSQ && SQM == 1;
  constexpr int SQ_CH = SQL ? BM * 8 / kThreads : 0;  // 16-byte chunks per thread per K step
  static_assert(!SQL || (SQ_CH >= 1 && SQ_CH * kThreads == BM * 8), "x tile chunks per thread");
  // Mode 0 with NSPLIT waves sharing x rows: each squares TI / NSPLIT of its
  // x subtiles.
  constexpr int NSPLIT = (WAVES_N < TI) ? WAVES_N : TI;
  constexpr bool SPLIT_SQ = SUMSQ && !SQL && NSPLIT >= 2 && (TI % NSPLIT) == 0 && (NSPLIT & (NSPLIT - 1)) == 0;
  constexpr int TSQ = SQL ? 0 : SPLIT_SQ ? TI / NSPLIT : TI;  // fragment slots 0 .. TSQ-1 are squared
  const int xsw = SPLIT_SQ ? (wn % NSPLIT) * TSQ : 0;  // slot i holds x subtile i ^ xsw
#pragma unroll
  for (int i = 0; i < TI; ++i) x_off[i] = wm * WTM + (i ^ xsw) * 32 + frow;

  // LayerNorm statistics are sums of x - sh over each row, sh = the row's
  // first element: xsh[i] for the rows of fragment slot i (which are also
  // the epilogue's rows), qsh[q] for the rows of the LDS-pass chunks.
  constexpr bool LNS = (EPI == EPI_LN) && SUMSQ;
  // Row statistics from a pass before the kernel (scale, and the LayerNorm
  // mean): requested here so their latency hides behind the K loop instead
  // of stalling every tile's epilogue.
  float pre_s[TI], pre_mu[TI];
  constexpr bool PRE = !SUMSQ && (EPI == EPI_PLAIN || EPI == EPI_LN || EPI == EPI_LATENT || F8);
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = min(m0 + x_off[i], M - 1);
      pre_s[i] = p.row_s != nullptr ? p.row_s[r] : 1.0f;
      pre_mu[i] = (EPI == EPI_LN && p.row_mu != nullptr) ? p.row_mu[r] : 0.f;
    }
  }
  // Head-norm gains of the lane's output columns (four consecutive per run
  // b of subtile j; v columns and columns past N take 1).  Where a wave has
  // at most two 32-column subtiles the registers allow them to be requested
  // here, so their latency hides behind the K loop; otherwise the epilogue
  // requests them.
  constexpr bool QKN = EPI == EPI_QKNORM || EPI == EPI_QKNORM_ROPE;
  constexpr bool EARLY_GAIN = QKN && TJ <= 2;
  f32x4 gain[QKN ? TJ : 1][4];
  auto load_gains = [&]() {
    if constexpr (QKN) {
      const int hd = p.head_dim;
      const int nq_heads = p.nq_cols / hd;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int c0 = n0 + (wn * TJ + j) * 32;  // first column of the subtile (wave-uniform)
        const bool is_q = c0 < p.nq_cols;
        const bool is_v = c0 >= p.nq_cols + p.nk_cols;
        const int head = c0 / hd;
        const float* gp =
            is_q ? p.g_q + (size_t)head * p.g_stride : p.g_k + (size_t)(is_v ? 0 : head - nq_heads) * p.g_stride;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int n = c0 + 8 * b + 4 * fchk;
          const int cih = n - head * hd;
          f32x4 g = {1.f, 1.f, 1.f, 1.f};
          if (!is_v && n < N) {  // N is a multiple of 4 here: all four columns exist
            if (p.g_vec4) {
              g = *reinterpret_cast<const f32x4*>(gp + cih);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) g[r] = gp[cih + r];
            }
          }
          gain[j][b] = g;
        }
      }
    }
  };
  if constexpr (EARLY_GAIN) load_gains();
  float xsh[TI];
  float qsh[SQ_CH > 0 ? SQ_CH : 1];
  if constexpr (LNS) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
      xsh[i] = __uint_as_float((uint32_t)p.A[(size_t)min(m0 + x_off[i], M - 1) * K] << 16);
    if constexpr (SQL) {
#pragma unroll
      for (int q = 0; q < SQ_CH; ++q)
        qsh[q] = __uint_as_float((uint32_t)p.A[(size_t)min(m0 + ((tid + q * kThreads) >> 3), M - 1) * K] << 16);
    }
  }

  // one MFMA sub-step worth of fragments: 16 bf16 values (32x32x16) or 64
  // fp8 values (32x32x64) of each operand row; lane l holds the FW 16-byte
  // chunks sub * 2 FW + FW (l / 32) + q, q < FW, of its row
  struct Frag {
    u32x4 w[TJ][FW], x[TI][FW];
  };
  auto read1 = [&](Frag& f, const uint16_t* sX, const uint16_t* sW, int sub) {
#pragma unroll
    for (int q = 0; q < FW; ++q) {
      const int chunk = sub * 2 * FW + fchk * FW + q;
#pragma unroll
      for (int j = 0; j < TJ; ++j) f.w[j][q] = *reinterpret_cast<const u32x4*>(sW + swz(w_off[j], chunk));
#pragma unroll
      for (int i = 0; i < TI; ++i) f.x[i][q] = *reinterpret_cast<const u32x4*>(sX + swz(x_off[i], chunk));
    }
  };

  f32x16 acc[TJ][TI];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;
  float ss[TI];  // only the first TSQ are used
  float s1[TI];  // LayerNorm: sums of x - sh
#pragma unroll
  for (int i = 0; i < TI; ++i) ss[i] = s1[i] = 0.f;

  auto mma1 = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if constexpr (F8) {
          // E4M3 for both operands (format selectors 0), no block scales
          const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(f.w[j][0], f.w[j][1], 0, 1, 2, 3, 4, 5, 6, 7));
          const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(f.x[i][0], f.x[i][1], 0, 1, 2, 3, 4, 5, 6, 7));
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j][i], 0, 0, 0, 0, 0, 0);
        } else {
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.w[j][0]),
                                                              __builtin_bit_cast(bf16x8, f.x[i][0]), acc[j][i], 0, 0, 0);
        }
      }
  };
  // mode 1: chunk q of this thread is row (tid + q kThreads) / 8 of the tile
  u32x4 sqv[SQ_CH > 0 ? SQ_CH : 1];
  float sqa[SQ_CH > 0 ? SQ_CH : 1];
  float sqb[SQ_CH > 0 ? SQ_CH : 1];  // LayerNorm: sums of x - sh
#pragma unroll
  for (int q = 0; q < (SQ_CH > 0 ? SQ_CH : 1); ++q) sqa[q] = sqb[q] = 0.f;
  auto sq_read = [&](const uint16_t* sX) {
    if constexpr (SQL) {
#pragma unroll
      for (int q = 0; q < SQ_CH; ++q) sqv[q] = *reinterpret_cast<const u32x4*>(sX + (tid + q * kThreads) * 8);
    }
  };
  auto sq_add = [&]() {
    if constexpr (SQL) {
#pragma unroll
      for (int q = 0; q < SQ_CH; ++q) {
        if constexpr (LNS)
          lnstat_bf16x8(sqv[q], qsh[q], sqb[q], sqa[q]);
        else
          sqa[q] = sumsq_bf16x8(sqv[q], sqa[q]);
      }
    }
  };
  auto square1 = [&](const Frag& f) {
    if constexpr (SUMSQ && !SQL) {
#pragma unroll
      for (int i = 0; i < TSQ; ++i) {
        if constexpr (LNS)
          lnstat_bf16x8(f.x[i][0], xsh[i], s1[i], ss[i]);
        else
          ss[i] = sumsq_bf16x8(f.x[i][0], ss[i]);
      }
    }
  };

  // ---- software pipeline --------------------------------------------------
  // A K step is four 16-wide sub-steps.  The fragments of sub-step s+1 are
  // read while the MFMAs of sub-step s run (two register sets).  Before the
  // last sub-step's MFMAs: wait for this wave's loads of tile kt+1, barrier
  // (tile kt+1 is then in the other stage for every wave, and stage c is no
  // longer read), read tile kt+1's first fragments and request tile kt+2
  // into stage c.  Scheduling hints interleave the reads, loads and VALU
  // squares with the MFMAs; sched_barrier keeps the sub-steps apart.
  Frag F[2];
  constexpr int NDS = (TJ + TI) * FW;  // fragment reads per sub-step
  constexpr int NMF = TJ * TI;  // MFMAs per sub-step
  constexpr int NLD = X_GROUPS + W_GROUPS;
  constexpr int NVA = TSQ * (LNS ? 32 : 16);  // square1() VALU ops
  // Interleave: one DS read before each MFMA while reads last, VALU work
  // spread over the MFMAs, then the loads.
  auto hints = [&](int nld, int nds, int nva) {
    const int vper = (nva + NMF - 1) / NMF;
#pragma unroll
    for (int k = 0; k < NMF; ++k) {
      if (k < nds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
      for (int v = 0; v < vper; ++v) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU
    }
    for (int k = NMF; k < nds; ++k) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    for (int k = 0; k < nld; ++k) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
  };
  // Every step has the same branch-free body.  Step kt reads stage kt % NS
  // and, once every wave is past its last read of it, refills it with tile
  // kt + NS.  Near the end that tile is clamped to the last one: the extra
  // loads land in a stage nobody reads again, and are waited for before LDS
  // is reused.
  auto step = [&](int kt, uint16_t* cX, uint16_t* cW, const uint16_t* nX, const uint16_t* nW) {
    sq_read(cX);
    read1(F[1], cX, cW, 1);
    mma1(F[0]);
    square1(F[0]);
    hints(0, SQ_CH + NDS, NVA);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NSUB == 4) {
      read1(F[0], cX, cW, 2);
      mma1(F[1]);
      square1(F[1]);
      sq_add();
      hints(0, NDS, NVA + (LNS ? 28 : 12) * SQ_CH);
      __builtin_amdgcn_sched_barrier(0);
      read1(F[1], cX, cW, 3);
      mma1(F[0]);
      square1(F[0]);
      hints(0, NDS, NVA);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (W3) {
      wait_vm<W_GROUPS>();  // tile kt+1 has landed (only weight tile kt+2 may be in flight)
    } else if constexpr (X3) {
      wait_vm<X_GROUPS>();  // tile kt+1 has landed (only x tile kt+2 may be in flight)
    } else {
      wait_vm<(NS - 2) * NLD>();  // this wave's part of tile kt+1 has landed
    }
    stage_barrier();  // ... and every wave's; stage c is free again
    __builtin_amdgcn_sched_barrier(0);
    read1(F[0], nX, nW, 0);
    if constexpr (W3) {
      issue_x(cX, min(kt + 2, KT - 1));
      issue_w(cW, min(kt + 3, KT - 1));
    } else if constexpr (X3) {
      issue_w(cW, min(kt + 2, KT - 1));
      issue_x(cX, min(kt + 3, KT - 1));
    } else {
      issue_tile(cX, cW, min(kt + NS, KT - 1));
    }
    mma1(F[1]);
    square1(F[1]);
    hints(NLD, NDS, NVA);
    __builtin_amdgcn_sched_barrier(0);
  };
  // fp8: a fragment is 32 bytes, and two full register sets of them do not
  // fit beside the 256 x 256 tile's accumulators.  So only the x fragments
  // are double-buffered (F[0].x / F[1].x); the weight fragments live in
  // F[0].w alone, and each is reloaded for the next sub-step as soon as the
  // MFMAs of the current one that read it have issued (a rolling reload).
  auto readx = [&](Frag& f, const uint16_t* sX, int sub) {
#pragma unroll
    for (int q = 0; q < FW; ++q)
#pragma unroll
      for (int i = 0; i < TI; ++i)
        f.x[i][q] = *reinterpret_cast<const u32x4*>(sX + swz(x_off[i], sub * 2 * FW + fchk * FW + q));
  };
  auto readw = [&](int j, const uint16_t* sW, int sub) {
#pragma unroll
    for (int q = 0; q < FW; ++q)
      F[0].w[j][q] = *reinterpret_cast<const u32x4*>(sW + swz(w_off[j], sub * 2 * FW + fchk * FW + q));
  };
  auto mma_roll = [&](const Frag& fx, const uint16_t* sW, int sub) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(F[0].w[j][0], F[0].w[j][FW - 1], 0, 1, 2,
                                                                            3, 4, 5, 6, 7));
        const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(fx.x[i][0], fx.x[i][FW - 1], 0, 1, 2, 3, 4,
                                                                            5, 6, 7));
        acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j][i], 0, 0, 0, 0, 0, 0);
      }
      readw(j, sW, sub);
    }
  };
  auto hints_roll = [&](int nld) {
    int xr = 0;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        if (xr < TI * FW) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read: an x fragment piece
          ++xr;
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x100, FW, 0);  // DS read: the weight fragment's reload
    }
    for (int k = 0; k < nld; ++k) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
  };
  auto step_roll = [&](int kt, uint16_t* cX, uint16_t* cW, const uint16_t* nX, const uint16_t* nW) {
    readx(F[1], cX, 1);
    mma_roll(F[0], cW, 1);
    hints_roll(0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (W3) {
      wait_vm<W_GROUPS>();
    } else {
      wait_vm<(NS - 2) * NLD>();
    }
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    readx(F[0], nX, 0);
    if constexpr (W3) {
      issue_x(cX, min(kt + 2, KT - 1));
      issue_w(cW, min(kt + 3, KT - 1));
    } else {
      issue_tile(cX, cW, min(kt + NS, KT - 1));
    }
    mma_roll(F[1], nW, 0);
    hints_roll(NLD);
    __builtin_amdgcn_sched_barrier(0);
  };
  // the rolling schedule for fp8 tiles with 256 rows (the others have the
  // registers for two full sets)
  constexpr bool ROLL = F8 && BM == 256;

  uint16_t* const sx[4] = {sx0, sx1, (NS > 2 || X3) ? sx2 : sx0, NS > 3 ? sx3 : sx0};
  uint16_t* const sw[4] = {sw0, sw1, (NS > 2 || W3) ? sw2 : sw0, NS > 3 ? sw3 : sw0};

#define FN_STEP(c)                                                                   \
  do {                                                                               \
    if constexpr (ROLL)                                                              \
      step_roll(kt, sx[c], sw[c], sx[((c) + 1) % NS], sw[((c) + 1) % NS]);           \
    else                                                                             \
      step(kt, sx[c], sw[c], sx[((c) + 1) % NS], sw[((c) + 1) % NS]);                \
  } while (0)
  // W3 ring: x stage kt % 2, weight stage kt % 3 (X3: the other way round)
#define FN_STEP3(q)                                                                  \
  do {                                                                               \
    if constexpr (X3)                                                                \
      step(kt, sx[(q) % 3], sw[(q) % 2], sx[((q) + 1) % 3], sw[((q) + 1) % 2]);      \
    else if constexpr (ROLL)                                                         \
      step_roll(kt, sx[(q) % 2], sw[(q) % 3], sx[((q) + 1) % 2], sw[((q) + 1) % 3]); \
    else                                                                             \
      step(kt, sx[(q) % 2], sw[(q) % 3], sx[((q) + 1) % 2], sw[((q) + 1) % 3]);      \
  } while (0)
  if (KT > 0) {
    if constexpr (W3) {
      issue_x(sx[0], 0);
      issue_w(sw[0], 0);
      issue_x(sx[1], min(1, KT - 1));
      issue_w(sw[1], min(1, KT - 1));
      issue_w(sw[2], min(2, KT - 1));
      wait_vm<X_GROUPS + 2 * W_GROUPS>();  // tile 0
    } else if constexpr (X3) {
      issue_x(sx[0], 0);
      issue_w(sw[0], 0);
      issue_x(sx[1], min(1, KT - 1));
      issue_w(sw[1], min(1, KT - 1));
      issue_x(sx[2], min(2, KT - 1));
      wait_vm<2 * X_GROUPS + W_GROUPS>();  // tile 0
    } else {
#pragma unroll
      for (int c = 0; c < NS; ++c) issue_tile(sx[c], sw[c], min(c, KT - 1));
      wait_vm<(NS - 1) * NLD>();  // tile 0
    }
    __syncthreads();
    if constexpr (ROLL) {
      readx(F[0], sX0, 0);
#pragma unroll
      for (int j = 0; j < TJ; ++j) readw(j, sW0, 0);
    } else {
      read1(F[0], sX0, sW0, 0);
    }
    int kt = 0;
    if constexpr (W3 || X3) {
      while (kt + 6 <= KT) {  // one operand's stages repeat every 2 steps, the other's every 3
        FN_STEP3(0); ++kt;
        FN_STEP3(1); ++kt;
        FN_STEP3(2); ++kt;
        FN_STEP3(3); ++kt;
        FN_STEP3(4); ++kt;
        FN_STEP3(5); ++kt;
      }
      if (kt < KT) { FN_STEP3(0); ++kt; }
      if (kt < KT) { FN_STEP3(1); ++kt; }
      if (kt < KT) { FN_STEP3(2); ++kt; }
      if (kt < KT) { FN_STEP3(3); ++kt; }
      if (kt < KT) { FN_STEP3(4); ++kt; }
    } else {
      while (kt + NS <= KT) {  // one pass over the NS stages
        FN_STEP(0);
        ++kt;
        FN_STEP(1);
        ++kt;
        if constexpr (NS > 2) {
          FN_STEP(2 % NS);
          ++kt;
        }
        if constexpr (NS > 3) {
          FN_STEP(3 % NS);
          ++kt;
        }
      }
      if (kt < KT) { FN_STEP(0); ++kt; }
      if (kt < KT) { FN_STEP(1 % NS); ++kt; }
      if constexpr (NS > 2) if (kt < KT) { FN_STEP(2 % NS); ++kt; }
    }
    wait_vm_all();  // the clamped loads of the last steps
  }
#undef FN_STEP
#undef FN_STEP3

  // ---- ragged last K step: masked register loads, then the same math -------
  if (k_tail) {
    __syncthreads();  // every wave is done with both stages
    const int kb = KT * BKE;  // first element of the tail
    constexpr int RPP = kThreads / 8;           // rows per pass
    const int lrow = tid >> 3, lchk = tid & 7;  // RPP rows x 8 chunks per pass
    const bool ok = kb + lchk * CE < K;         // K is a whole number of chunks
    const int lv = (lrow * K + lchk * CE + kb) * EB;
    const int pass_bytes = RPP * K * EB;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < (BM + RPP - 1) / RPP; ++i) {
      if (i * RPP + lrow < BM) {
        const u32x4 v = ok ? __builtin_amdgcn_raw_buffer_load_b128(rs_x, lv, i * pass_bytes, 0) : z;
        *reinterpret_cast<u32x4*>(sX0 + swz(i * RPP + lrow, lchk)) = v;
      }
    }
    static_assert(BN % (2 * RPP) == 0, "whole passes over each weight half");
#pragma unroll
    for (int i = 0; i < BN / RPP; ++i) {
      u32x4 v = z;
      if (ok) {
        if constexpr (EPI == EPI_GLU) {
          constexpr int HALF = BN / 2 / RPP;  // passes over gate rows
          v = (i < HALF) ? __builtin_amdgcn_raw_buffer_load_b128(rs_w0, lv, i * pass_bytes, 0)
                         : __builtin_amdgcn_raw_buffer_load_b128(rs_w1, lv, (i - HALF) * pass_bytes, 0);
        } else {
          v = __builtin_amdgcn_raw_buffer_load_b128(rs_w0, lv, i * pass_bytes, 0);
        }
      }
      *reinterpret_cast<u32x4*>(sW0 + swz(i * RPP + lrow, lchk)) = v;
    }
    __syncthreads();
    sq_read(sX0);
    sq_add();
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      read1(F[0], sX0, sW0, sub);
      mma1(F[0]);
      square1(F[0]);
    }
  }

  // ---- epilogue ------------------------------------------------------------
  // Lane l holds, for x subtile i, output row m = m0 + wm WTM + 32 i + l % 32
  // and, for W* subtile j and run b, columns 8 b + 4 (l / 32) + (0..3) of the
  // subtile.  Its own squares plus its partner lane's (l ^ 32) give s[m].
  float srow[TI];
  float mrow[TI];  // LayerNorm row mean (0 otherwise)
  // Row totals -> scale (and mean).  LayerNorm: the zero columns past K in
  // the last K step each added -sh and sh^2; take them out, then
  // mean = sh + S1/K, var = S2/K - (S1/K)^2.
  const int kpad = (KT + (k_tail ? 1 : 0)) * BKE - K;
  auto row_stat = [&](int i, float t2, float t1) {
    if constexpr (LNS) {
      const float sh = xsh[i];
      t1 = fmaf((float)kpad, sh, t1);
      t2 = fmaf(-(float)kpad * sh, sh, t2);
      const float md = t1 * p.inv_k;
      const float var = fmaxf(fmaf(-md, md, t2 * p.inv_k), 0.f);
      mrow[i] = sh + md;
      return rsqrtf(var + p.eps);
    } else {
      mrow[i] = 0.f;
      return rsqrtf(t2 * p.inv_k + p.eps);
    }
  };
  if constexpr (SQL) {
    // the 8 threads of a row are 8 consecutive lanes; their sums meet in LDS
    float* const sq_x = reinterpret_cast<float*>(sx0);  // [BM] sums of squares, then [BM] LayerNorm sums
    float t[SQ_CH], tb[SQ_CH];
#pragma unroll
    for (int q = 0; q < SQ_CH; ++q) {
      t[q] = xor_sum<4>(xor_sum<2>(xor_sum<1>(sqa[q])));
      if constexpr (LNS) tb[q] = xor_sum<4>(xor_sum<2>(xor_sum<1>(sqb[q])));
    }
    __syncthreads();
    if ((tid & 7) == 0) {
#pragma unroll
      for (int q = 0; q < SQ_CH; ++q) {
        sq_x[(tid + q * kThreads) >> 3] = t[q];
        if constexpr (LNS) sq_x[BM + ((tid + q * kThreads) >> 3)] = tb[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = wm * WTM + i * 32 + frow;
      srow[i] = row_stat(i, sq_x[r], LNS ? sq_x[BM + r] : 0.f);
    }
  } else if constexpr (SPLIT_SQ) {
    // slots 0 .. TSQ-1 hold this wave's own sums; the others come from the
    // waves with other values of wn % NSPLIT, through stage 0 of LDS (idle
    // now: every wave is past its last fragment read).  Waves with the same
    // wn % NSPLIT write identical sums.
    float* const sq_x = reinterpret_cast<float*>(sx0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TSQ; ++i) {
      const float own = xor_sum<32>(ss[i]);
      const float own1 = LNS ? xor_sum<32>(s1[i]) : 0.f;
      if (fchk == 0) {
        sq_x[wm * WTM + (i ^ xsw) * 32 + frow] = own;
        if constexpr (LNS) sq_x[BM + wm * WTM + (i ^ xsw) * 32 + frow] = own1;
      }
      srow[i] = row_stat(i, own, own1);
    }
    __syncthreads();
#pragma unroll
    for (int i = TSQ; i < TI; ++i) {
      const int r = wm * WTM + (i ^ xsw) * 32 + frow;
      srow[i] = row_stat(i, sq_x[r], LNS ? sq_x[BM + r] : 0.f);
    }
  } else {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      if constexpr (SUMSQ) {
        const float t = xor_sum<32>(ss[i]);
        srow[i] = row_stat(i, t, LNS ? xor_sum<32>(s1[i]) : 0.f);
      } else if constexpr (PRE) {
        srow[i] = pre_s[i];  // from a pass before the kernel, if any (1 and 0 otherwise)
        mrow[i] = pre_mu[i];
      } else {
        srow[i] = 1.0f;
        mrow[i] = 0.f;
      }
    }
  }

  using OutT = typename std::conditional<OUT_BF16, uint16_t, float>::type;
  OutT* const Y = static_cast<OutT*>(p.Y);
  const bool fast = (m0 + BM <= M) && (n0 + OUT_BN <= N) && ((N & 3) == 0);
  auto store4 = [&](int m, int n, const float v[4]) {  // row m, columns n..n+3
    if (fast) {
      if constexpr (OUT_BF16) {
        uint2 u;
        u.x = pack_bf16x2(v[0], v[1]);
        u.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(Y + (size_t)m * N + n) = u;
      } else {
        *reinterpret_cast<float4*>(Y + (size_t)m * N + n) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else if (m < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) {
          if constexpr (OUT_BF16)
            Y[(size_t)m * N + n + r] = out_bf16_bits(v[r]);
          else
            Y[(size_t)m * N + n + r] = v[r];
        }
    }
  };
  auto row_of = [&](int i) { return m0 + wm * WTM + (i ^ xsw) * 32 + frow; };
  auto col_of = [&](int j, int b) { return n0 + wn * WOUT + j * 32 + 8 * b + 4 * fchk; };

  // bf16 output of an interior tile goes through LDS: each wave writes its
  // WTM x WOUT block there (16-byte chunk c of block row r at slot
  // c ^ (r % CPR)), then stores whole row segments, 16 bytes per lane, so
  // every global store fills complete cache lines.
  constexpr int RS = WOUT * 2;   // bytes per block row
  constexpr int CPR = RS / 16;   // 16-byte chunks per block row
  constexpr int BLK = WTM * RS;  // bytes per wave block
  constexpr int BPX = (XE * 2) / BLK, BPW = (WE * 2) / BLK;  // blocks per x / W* stage object
  constexpr bool CAN_STAGE = OUT_BF16 && EPI != EPI_LATENT && CPR >= 4 && NS * (BPX + BPW) >= kWaves &&
                             (WTM * CPR) % 64 == 0;
  const bool staged = CAN_STAGE && fast && (N % 8) == 0;  // tile-uniform
  uint8_t* blk = nullptr;
  if constexpr (CAN_STAGE) {
    // wave w takes block w of the list: the W* stages' blocks, then the x stages'
    uint16_t* const objs[8] = {sw[0], sw[1], sw[2], sw[3], sx[0], sx[1], sx[2], sx[3]};
    int b = wave;
#pragma unroll
    for (int o = 0; o < 2 * NS; ++o) {
      const int per = o < NS ? BPW : BPX;
      uint16_t* const obj = objs[o < NS ? o : 4 + (o - NS)];
      if (blk == nullptr && b < per) blk = reinterpret_cast<uint8_t*>(obj) + b * BLK;
      if (blk == nullptr) b -= per;
    }
  }
  auto emit = [&](int i, int j, int b, const float v[4]) {
    if (staged) {
      const int r = (i ^ xsw) * 32 + frow;
      const int c = j * 4 + b;
      uint2 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(blk + r * RS + ((c ^ (r % CPR)) << 4) + fchk * 8) = u;
    } else {
      store4(row_of(i), col_of(j, b), v);
    }
  };
  auto flush = [&]() {
    if constexpr (CAN_STAGE) {
      if (staged) {  // the wave reads back only its own writes: LDS keeps their order
        const size_t row0 = (size_t)m0 + wm * WTM;
        const int col0 = n0 + wn * WOUT;
#pragma unroll
        for (int it = 0; it < WTM * CPR / 64; ++it) {
          const int idx = it * 64 + lane;
          const int r = idx / CPR, c = idx % CPR;
          const u32x4 d = *reinterpret_cast<const u32x4*>(blk + r * RS + ((c ^ (r % CPR)) << 4));
          *reinterpret_cast<u32x4*>(Y + (row0 + r) * N + col0 + c * 8) = d;
        }
      }
    }
  };

  // fp8: the weight's channel scales of the tile's columns (gate, then up
  // for glu), read once per tile into LDS of their own (one 16-byte load
  // per thread), then read per run: 64 registers of them would not fit
  // beside the accumulators.
  constexpr int NCQ = F8 ? (EPI == EPI_GLU ? 2 : 1) * OUT_BN : 4;
  __shared__ __attribute__((aligned(16))) float colq_lds[NCQ];
  if constexpr (F8) {
    static_assert(NCQ / 4 <= kThreads, "one vector per thread");
    if (tid < NCQ / 4) {
      const int which = tid / (OUT_BN / 4), q4 = tid % (OUT_BN / 4);
      const float* q = which == 0 ? p.col_q0 : p.col_q1;
      const int n = n0 + 4 * q4;
      f32x4 r = {1.f, 1.f, 1.f, 1.f};
      if (n + 3 < N) {
        r = *reinterpret_cast<const f32x4*>(q + n);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (n + c < N) r[c] = q[n + c];
      }
      *reinterpret_cast<f32x4*>(colq_lds + which * OUT_BN + 4 * q4) = r;
    }
    __syncthreads();
  }
  auto colq4 = [&](int which, int n) { return *reinterpret_cast<const f32x4*>(colq_lds + which * OUT_BN + (n - n0)); };
  if constexpr (EPI == EPI_PLAIN) {
    if (staged) __syncthreads();  // every wave is done with LDS
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float v[4];
          f32x4 cq = {1.f, 1.f, 1.f, 1.f};
          if constexpr (F8) cq = colq4(0, col_of(j, b));
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[j][i][4 * b + r] * srow[i] * cq[r];
          emit(i, j, b, v);
        }
    flush();
  } else if constexpr (EPI == EPI_GLU) {
    if (staged) __syncthreads();
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ / 2; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float v[4];
          f32x4 cg = {1.f, 1.f, 1.f, 1.f}, cu = {1.f, 1.f, 1.f, 1.f};
          if constexpr (F8) {
            cg = colq4(0, col_of(j, b));
            cu = colq4(1, col_of(j, b));
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = acc[j][i][4 * b + r] * srow[i] * cg[r];
            const float u = acc[j + TJ / 2][i][4 * b + r] * srow[i] * cu[r];
            v[r] = silu(a) * u;
          }
          emit(i, j, b, v);
        }
    flush();
  } else if constexpr (EPI == EPI_LN) {
    // y = s (z - mu c[n]) + b[n].  The tile's column sums and biases are
    // read once into LDS (one global load per thread, N-tail columns one by
    // one), so the epilogue waits for memory once, not once per subtile.
    // Own LDS when it fits beside the stages without costing a workgroup
    // per CU; else a stage the staged stores never use (the W3 ring's third
    // weight stage, or the last x stage when the blocks before it hold every
    // wave's output block).
    static_assert(OUT_BN / 2 <= kThreads, "one vector per thread");
    constexpr int LDS_CU = 160 * 1024;
    constexpr int STAGE_BYTES = NS * (XE + WE) * 2 + (W3 ? WE * 2 : 0);
    constexpr bool OWN = LDS_CU / (STAGE_BYTES + OUT_BN * 8) == LDS_CU / STAGE_BYTES;
    constexpr bool LAST_X_FREE = !CAN_STAGE || (NS * BPW + (NS - 1) * BPX >= kWaves);
    static_assert(OWN || W3 || (LAST_X_FREE && XE * 2 >= OUT_BN * 8), "room for the column vectors");
    __shared__ f32x4 lncb_own[OWN ? OUT_BN / 2 : 1];
    f32x4* lncb0;
    if constexpr (OWN) {
      lncb0 = lncb_own;
    } else {
      lncb0 = reinterpret_cast<f32x4*>(W3 ? sw[2] : sx[NS - 1]);
      __syncthreads();  // every wave is past its last fragment read of that stage
    }
    f32x4* const lncb[2] = {lncb0, lncb0 + OUT_BN / 4};
    const bool use_c = LNS || p.row_mu != nullptr;
    if (tid < OUT_BN / 2) {
      const int which = tid / (OUT_BN / 4), q4 = tid % (OUT_BN / 4);
      const float* v = which == 0 ? (use_c ? p.ln_c : nullptr) : p.ln_b;
      const int n = n0 + 4 * q4;
      f32x4 r = {0.f, 0.f, 0.f, 0.f};
      if (v != nullptr) {
        if (n + 3 < N) {
          r = *reinterpret_cast<const f32x4*>(v + n);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) r[q] = v[n + q];
        }
      }
      lncb[which][q4] = r;
    }
    __syncthreads();  // also: every wave is done with the stages (staged stores)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int q4 = (col_of(j, b) - n0) >> 2;
          const f32x4 cc = lncb[0][q4], bb = lncb[1][q4];
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = fmaf(fmaf(-mrow[i], cc[r], acc[j][i][4 * b + r]), srow[i], bb[r]);
          emit(i, j, b, v);
        }
    flush();
  } else if constexpr (EPI == EPI_LATENT) {
    // Latent subtiles (wave-uniform: lat_cols % 32 == 0) store the unscaled
    // product to the float32 workspace and each row's sum of squares over
    // the 32 columns (the lane's 16 values plus its partner lane's); a
    // latent spans several tiles, so a row kernel applies its norm.  The
    // columns after the latents: z * s[m], then the rotation of the row's
    // position when positions are given (a position outside the table
    // gives NaN).
    const int lat = p.lat_cols;
    const int lat_subs = lat / 32;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int m = row_of(i);
      int pos = 0;
      bool pos_ok = false;
      if (p.pos != nullptr) {
        pos = p.pos[min(m, M - 1)];
        pos_ok = pos >= 0 && pos < p.n_pos;
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int c0 = n0 + (wn * TJ + j) * 32;
        if (c0 < lat) {
          float ssq = 0.f;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              v[r] = acc[j][i][4 * b + r];
              ssq = fmaf(v[r], v[r], ssq);
            }
            if (m < M) *reinterpret_cast<f32x4*>(p.lat_z + (size_t)m * lat + col_of(j, b)) = v;
          }
          ssq = xor_sum<32>(ssq);
          if (fchk == 0 && m < M) p.lat_part[(size_t)m * lat_subs + c0 / 32] = ssq;
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int n = col_of(j, b);
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[j][i][4 * b + r] * srow[i];
            const int cih = n - lat;
            if (p.pos != nullptr && n < N && cih < p.rot_dim) {
              const float qnan = __builtin_nanf("");
              const f32x4 c = pos_ok ? *reinterpret_cast<const f32x4*>(p.rope + (size_t)pos * p.rot_dim + cih)
                                     : f32x4{qnan, qnan, qnan, qnan};
              const float a0 = v[0], b0 = v[1], a1 = v[2], b1 = v[3];
              v[0] = a0 * c[0] - b0 * c[1];
              v[1] = a0 * c[1] + b0 * c[0];
              v[2] = a1 * c[2] - b1 * c[3];
              v[3] = a1 * c[3] + b1 * c[2];
            }
            store4(m, n, v);
          }
        }
      }
    }
  } else {  // EPI_QKNORM, EPI_QKNORM_ROPE
    // Head sums of z^2 per row: the lane's 16 values of a subtile, plus its
    // partner lane's, give the 32-column sum; subtile sums meet in LDS so a
    // head spanning several waves is summed across them.
    constexpr bool ROPE = EPI == EPI_QKNORM_ROPE;
    constexpr int SUBS = BN / 32;
    static_assert(BM * SUBS * 4 <= XE * 2, "partials fit in the first x stage");
    const int hd = p.head_dim;
    const int subs_per_head = hd / 32;
    // the gains, if not requested before the K loop: before the barriers,
    // so their latency overlaps the head sums
    if constexpr (!EARLY_GAIN) load_gains();
    // token positions of this lane's rows (rows past the end read the last row)
    int rpos[TI];
    if constexpr (ROPE) {
#pragma unroll
      for (int i = 0; i < TI; ++i) rpos[i] = p.pos[min(row_of(i), M - 1)];
    }
    float* part = reinterpret_cast<float*>(sx0);  // [BM][SUBS]; stages are idle now
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        float v = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) v += acc[j][i][e] * acc[j][i][e];
        v = xor_sum<32>(v);
        if (fchk == 0) part[(wm * WTM + (i ^ xsw) * 32 + frow) * SUBS + wn * TJ + j] = v;
      }
    __syncthreads();
    float scale[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int trow = wm * WTM + (i ^ xsw) * 32 + frow;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int sub = wn * TJ + j;
        const int c0 = n0 + sub * 32;
        const bool is_v = c0 >= p.nq_cols + p.nk_cols;
        scale[i][j] = srow[i];
        if (!(is_v && p.v_mode == 0)) {
          const int hfirst = (sub / subs_per_head) * subs_per_head;
          float hs = 0.f;
          for (int q = 0; q < subs_per_head; ++q) hs += part[trow * SUBS + hfirst + q];
          scale[i][j] = rsqrtf(hs / (float)hd + p.eps_head);
        }
      }
    }
    if (staged) __syncthreads();  // the head partials are no longer needed
    if constexpr (ROPE) {
      // scale and gain go into the accumulators first, so the gain
      // registers are free before the rotary table loads
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[j][i][e] = acc[j][i][e] * scale[i][j] * gain[j][e / 4][e % 4];
    }
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      // Rotary embedding after the gain: the lane's four consecutive columns
      // c..c+3 of a head (c % 4 == 0) are pairs c/2 and c/2 + 1, whose
      // (cos, sin) sit at t[pos * rot_dim + c .. + 3].  Columns past rot_dim
      // and v heads keep (cos, sin) = (1, 0); a position outside the table
      // gives NaN.  The load itself always stays inside the table (position
      // and column clamped) and is issued per subtile, which keeps the
      // 256-row tile within its registers.
      const bool pos_ok = !ROPE || (rpos[i] >= 0 && rpos[i] < p.n_pos);
      const float* trow = ROPE ? p.rope + (size_t)(pos_ok ? rpos[i] : 0) * p.rot_dim : nullptr;
      const float qnan = __builtin_nanf("");
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        f32x4 cs[4];
        if constexpr (ROPE) {
          const int c0 = n0 + (wn * TJ + j) * 32;
          const bool is_qk = c0 < p.nq_cols + p.nk_cols;
          const int head = c0 / hd;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int cih = col_of(j, b) - head * hd;
            const f32x4 t = *reinterpret_cast<const f32x4*>(trow + min(cih, p.rot_dim - 4));
            const bool rot = is_qk && cih < p.rot_dim;
            f32x4 c;
            c[0] = rot ? (pos_ok ? t[0] : qnan) : 1.f;
            c[1] = rot ? (pos_ok ? t[1] : qnan) : 0.f;
            c[2] = rot ? (pos_ok ? t[2] : qnan) : 1.f;
            c[3] = rot ? (pos_ok ? t[3] : qnan) : 0.f;
            cs[b] = c;
          }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float v[4];
          if constexpr (ROPE) {
            const f32x4 c = cs[b];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[j][i][4 * b + r];
            const float a0 = v[0], b0 = v[1], a1 = v[2], b1 = v[3];
            v[0] = a0 * c[0] - b0 * c[1];
            v[1] = a0 * c[1] + b0 * c[0];
            v[2] = a1 * c[2] - b1 * c[3];
            v[3] = a1 * c[3] + b1 * c[2];
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[j][i][4 * b + r] * scale[i][j] * gain[j][b][r];
          }
          emit(i, j, b, v);
        }
      }
    }
    flush();
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NS, int SQM, int EPI, bool SUMSQ, bool OUT_BF16,
          bool W3 = false, bool F8 = false, bool X3 = false>
hipError_t launch_cfg(const GemmArgs& a0, hipStream_t st) {
  GemmArgs a = a0;
  constexpr int OUT_BN = (EPI == EPI_GLU) ? BN / 2 : BN;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + OUT_BN - 1) / OUT_BN;
  if (a.group_m <= 0) a.group_m = 8;
  const int nblk = a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WAVES_M, WAVES_N, NS, SQM, W3, EPI, SUMSQ, OUT_BF16, F8, X3>),
                     dim3(nblk), dim3(WAVES_M * WAVES_N * 64), 0, st, a);
  return hipGetLastError();
}

template <int EPI, bool SUMSQ, bool OUT_BF16>
hipError_t launch_tile(int tile, const GemmArgs& a, hipStream_t st) {
  switch (tile) {
    case TILE_256x256:    return launch_cfg<256, 256, 4, 2, 2, 0, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_128x256:    return launch_cfg<128, 256, 2, 4, 2, 0, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_64x256:     return launch_cfg<64, 256, 2, 4, 2, 0, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_128x128:    return launch_cfg<128, 128, 4, 2, 2, 0, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_128x256_S3: return launch_cfg<128, 256, 2, 4, 3, 0, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_64x256_S4Q: return launch_cfg<64, 256, 2, 4, 4, 1, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_256x256_Q:  return launch_cfg<256, 256, 4, 2, 2, 1, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_128x128_Q:  return launch_cfg<128, 128, 4, 2, 2, 1, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_256x256_W3: return launch_cfg<256, 256, 4, 2, 2, 0, EPI, SUMSQ, OUT_BF16, true>(a, st);
    case TILE_256x256_X3:
      if constexpr (EPI == EPI_PLAIN)
        return launch_cfg<256, 256, 4, 2, 2, 0, EPI, SUMSQ, OUT_BF16, false, false, true>(a, st);
      else
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// fp8 tiles (E4M3 x and weights; the row statistics come from the pass
// that quantises x, so no squares).  The four-stage 64-row tile and the
// three-stage weight ring of the 256-row tile leave no LDS for the channel
// scales (and the ring spills), so they are not built for fp8.
template <int EPI, bool OUT_BF16>
hipError_t launch_tile_f8(int tile, const GemmArgs& a, hipStream_t st) {
  switch (tile) {
    case TILE_256x256:    return launch_cfg<256, 256, 4, 2, 2, 0, EPI, false, OUT_BF16, false, true>(a, st);
    case TILE_128x256:    return launch_cfg<128, 256, 2, 4, 2, 0, EPI, false, OUT_BF16, false, true>(a, st);
    case TILE_128x128:    return launch_cfg<128, 128, 4, 2, 2, 0, EPI, false, OUT_BF16, false, true>(a, st);
    case TILE_128x256_S3: return launch_cfg<128, 256, 2, 4, 3, 0, EPI, false, OUT_BF16, false, true>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// One translation unit per epilogue (the build compiles this file once for
// each FN_GEMM_EPI value), so the instantiations compile in parallel.
#ifndef FN_GEMM_EPI
#error "compile with -DFN_GEMM_EPI=<Epi value>"
#endif

template <>
hipError_t launch_gemm_bf16_epi<FN_GEMM_EPI>(bool sumsq, bool out_bf16, int tile, const GemmArgs& a, hipStream_t st) {
  constexpr int E = FN_GEMM_EPI;
  if (sumsq) return out_bf16 ? launch_tile<E, true, true>(tile, a, st) : launch_tile<E, true, false>(tile, a, st);
  return out_bf16 ? launch_tile<E, false, true>(tile, a, st) : launch_tile<E, false, false>(tile, a, st);
}

#if FN_GEMM_EPI == 0 || FN_GEMM_EPI == 1
template <>
hipError_t launch_gemm_fp8_epi<FN_GEMM_EPI>(bool out_bf16, int tile, const GemmArgs& a, hipStream_t st) {
  constexpr int E = FN_GEMM_EPI;
  return out_bf16 ? launch_tile_f8<E, true>(tile, a, st) : launch_tile_f8<E, false>(tile, a, st);
}
#endif

}  // namespace fn
