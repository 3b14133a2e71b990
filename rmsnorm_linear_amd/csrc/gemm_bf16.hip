// Prefill kernel: bf16 MFMA contraction with the row sum of squares taken
// from the same x fragments that feed the matrix cores, and the deferred row
// scale applied in the epilogue (FlashNorm Abstract, points (i) and (ii)).
//
//   C[m, n] = sum_k A[m, k] * B[n, k]     A = x [M x K], B = W* [N x K], both
//                                          K-contiguous bf16; fp32 accumulate
//   ss[m]   = sum_k A[m, k]^2              VALU, from the A fragments
//   s[m]    = 1 / sqrt(ss[m] / K + eps)
//   epilogue: plain  y = C * s
//             glu    h = SiLU(s * C_gate) * (s * C_up)
//             qknorm per-head RMSNorm of C on q/k heads, v = C * s (or normed)
//
// Layout and pipeline (gfx950):
//  * Workgroup tile BM x BN, K step 64, 4 waves (WAVES_M x WAVES_N); each
//    wave owns a (BM/WAVES_M) x (BN/WAVES_N) block of 32x32 accumulators
//    (v_mfma_f32_32x32x16_bf16: on gfx950 one wave per SIMD keeps the matrix
//    core far busier with the 32x32 shape than with 16x16x32).
//  * Operands stream HBM -> LDS with buffer_load_dwordx4 ... lds (no staging
//    registers): each load instruction fills 8 rows x 128 B of a stage.  A
//    stage keeps rows of 64 bf16 (128 B) with the eight 16-byte chunks of
//    row r stored at slot (chunk ^ (r % 8)), so a fragment read of 8
//    consecutive rows touches 8 different bank groups; the loads pick the
//    global chunk per lane so the bytes land in that swizzled order.
//  * Two LDS stages, one barrier per K step.  Fragments are double-buffered
//    in registers: the second half-step's fragments are read while the
//    first half's MFMAs run, and the next tile's first fragments are read
//    (and the tile after next is requested from HBM) while the second
//    half's MFMAs run.
//  * Buffer resources start at the tile's first row and end at the
//    tensor's last row, so rows past M or N read as zeros.  A ragged last K
//    step (K % 64 != 0) goes through registers with lane masks, after the
//    pipelined loop.
//  * Every x element is squared once per workgroup: the waves sharing a row
//    block split its fragments between them and combine through LDS.

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace fn {

namespace {

constexpr int BK = 64;
constexpr int kThreads = 256;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI, bool SUMSQ, bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int WM = BM / WAVES_M;
  constexpr int WN = BN / WAVES_N;
  constexpr int TM = WM / 32;
  constexpr int TN = WN / 32;
  constexpr int A_GROUPS = BM / 8 / 4;  // 8-row load groups per wave
  constexpr int B_GROUPS = BN / 8 / 4;
  static_assert(WAVES_M * WAVES_N == 4, "4 waves");
  static_assert(EPI != EPI_GLU || (TN % 2) == 0, "glu pairs gate/up subtiles");

  // Two operand stages (A and B tiles each), separate objects so the
  // compiler can tell a fragment read of one stage from an in-flight
  // direct-to-LDS load into the other (and need not wait for the load).
  // The epilogue reuses both.
  __shared__ __attribute__((aligned(16))) uint16_t st0[(BM + BN) * BK];
  __shared__ __attribute__((aligned(16))) uint16_t st1[(BM + BN) * BK];
  __shared__ float srow_lds[BM];
  uint16_t* const sA0 = st0;
  uint16_t* const sB0 = st0 + BM * BK;
  uint16_t* const sA1 = st1;
  uint16_t* const sB1 = st1 + BM * BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

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
  constexpr int OUT_BN = (EPI == EPI_GLU) ? BN / 2 : BN;  // output columns per tile
  const int n0 = tile_n * OUT_BN;

  const int M = p.M, K = p.K, N = p.N;
  const int KT = K / BK;  // full K steps
  const bool k_tail = (K % BK) != 0;

  // ---- buffer resources ----------------------------------------------------
  auto make_rsrc = [&](const uint16_t* base, int rows_left) {
    const int64_t bytes = (int64_t)rows_left * K * 2;
    const int nrec = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nrec, 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.A + (size_t)m0 * K, M - m0);
  const __amdgpu_buffer_rsrc_t rs_b0 = make_rsrc(p.B0 + (size_t)n0 * K, N - n0);
  const __amdgpu_buffer_rsrc_t rs_b1 = (EPI == EPI_GLU) ? make_rsrc(p.B1 + (size_t)n0 * K, N - n0) : rs_b0;

  // Direct loads: lane l of a group fills LDS slot l % 8 of row l / 8, which
  // holds global chunk (l % 8) ^ (l / 8) of that row.
  const int g_row = lane >> 3;
  const int g_chunk = (lane & 7) ^ g_row;
  const int voff = (g_row * K + g_chunk * 8) * 2;
  const int group_bytes = 8 * K * 2;

  auto issue_tile = [&](uint16_t* sA, uint16_t* sB, int kt) {
    const int kb = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < A_GROUPS; ++i) {
      const int g = wave * A_GROUPS + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void*)(sA + g * 8 * BK), 16, voff, g * group_bytes + kb, 0,
                                               0);
    }
#pragma unroll
    for (int i = 0; i < B_GROUPS; ++i) {
      const int g = wave * B_GROUPS + i;
      if constexpr (EPI == EPI_GLU) {
        constexpr int HALF = BN / 16;  // groups of gate rows
        if (g < HALF)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b0, (lds_void*)(sB + g * 8 * BK), 16, voff,
                                                   g * group_bytes + kb, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b1, (lds_void*)(sB + g * 8 * BK), 16, voff,
                                                   (g - HALF) * group_bytes + kb, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b0, (lds_void*)(sB + g * 8 * BK), 16, voff, g * group_bytes + kb,
                                                 0, 0);
      }
    }
  };

  // ---- fragments -------------------------------------------------------------
  // 32x32x16 operands: lane l holds row (or column) l % 32 of a subtile and
  // the 8-element K chunk l / 32 of the 16-wide K sub-step.  A K step of 64 is
  // four sub-steps; fragments come in pairs of sub-steps (halves 0 and 1).
  const int frow = lane & 31;
  const int fchk = lane >> 5;
  int a_off[TM], b_off[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_off[i] = wm * WM + i * 32 + frow;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if constexpr (EPI == EPI_GLU)
      b_off[j] = (j < TN / 2) ? wn * (WN / 2) + j * 32 + frow : BN / 2 + wn * (WN / 2) + (j - TN / 2) * 32 + frow;
    else
      b_off[j] = wn * WN + j * 32 + frow;
  }

  struct Frags {
    u32x4 a[2][TM], b[2][TN];
  };
  auto read_frags = [&](Frags& f, const uint16_t* sA, const uint16_t* sB, int half) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int chunk = (half * 2 + s2) * 2 + fchk;
#pragma unroll
      for (int i = 0; i < TM; ++i) f.a[s2][i] = *reinterpret_cast<const u32x4*>(sA + swz(a_off[i], chunk));
#pragma unroll
      for (int j = 0; j < TN; ++j) f.b[s2][j] = *reinterpret_cast<const u32x4*>(sB + swz(b_off[j], chunk));
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // this wave squares A subtiles i with i % WAVES_N == wn
  constexpr int SQ = (TM + WAVES_N - 1) / WAVES_N;
  float ss[SQ];
#pragma unroll
  for (int q = 0; q < SQ; ++q) ss[q] = 0.f;

  auto mma = [&](const Frags& f, int s2) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a[s2][i]),
                                                            __builtin_bit_cast(bf16x8, f.b[s2][j]), acc[i][j], 0, 0, 0);
  };
  // The subtile a wave squares is picked with selects on the wave-uniform
  // index (no branches), so the scheduler can spread the VALU work between
  // MFMAs.  Waves that own no subtile (TM < WAVES_N) square a duplicate that
  // is never published.
  auto pick = [&](const u32x4* arr, int q) {
    u32x4 v = arr[q * WAVES_N];
#pragma unroll
    for (int w = 1; w < WAVES_N; ++w)
      if (q * WAVES_N + w < TM) v = (wn == w) ? arr[q * WAVES_N + w] : v;
    return v;
  };
  auto square = [&](const Frags& f) {
    if constexpr (SUMSQ) {
#pragma unroll
      for (int q = 0; q < SQ; ++q) {
        ss[q] = sumsq_bf16x8(pick(f.a[0], q), ss[q]);
        ss[q] = sumsq_bf16x8(pick(f.a[1], q), ss[q]);
      }
    }
  };

  // One K step on stage (cA, cB) with the next tile in (nA, nB).
  //   region 1: read the second-half fragments, first-half MFMAs, squares
  //   barrier (tile kt+1 has landed in the other stage; stage c is free)
  //   region 2: read tile kt+1's first fragments, request tile kt+2 into
  //             stage c, second-half MFMAs
  // Scheduling hints interleave LDS reads, buffer loads and VALU work with
  // the MFMAs of each region; sched_barrier keeps the regions apart.
  Frags F0, F1;
  constexpr int NDS = 2 * (TM + TN);  // fragment reads per half
  constexpr int NMF = 2 * TM * TN;    // MFMAs per half
  constexpr int NLD = A_GROUPS + B_GROUPS;
  constexpr int NVA = SUMSQ ? 2 * SQ * 2 * (4 * (WAVES_N - 1) + 16) : 0;  // square() VALU ops
  constexpr int VPER = (NVA + (NMF - NDS / 2) - 1) / (NMF - NDS / 2);
  auto hints_region1 = [&]() {
#pragma unroll
    for (int k = 0; k < NDS / 2; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
#pragma unroll
    for (int k = 0; k < NMF - NDS / 2; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (VPER > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);  // VALU
    }
  };
  auto hints_region2 = [&]() {
    // every fragment read is issued before the first direct-to-LDS load
#pragma unroll
    for (int k = 0; k < NDS / 2; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    }
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  // Every step has the same branch-free body.  Near the end the "next" and
  // "after next" tiles are clamped to the last tile: the extra loads land in
  // a stage nobody reads again, and are waited for before LDS is reused.
  auto step = [&](int kt, uint16_t* cA, uint16_t* cB, const uint16_t* nA, const uint16_t* nB) {
    read_frags(F1, cA, cB, 1);
    mma(F0, 0);
    mma(F0, 1);
    square(F0);
    square(F1);
    hints_region1();
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_all();    // this wave's part of tile kt+1 has landed
    __syncthreads();  // ... and every wave's; stage c is free again
    __builtin_amdgcn_sched_barrier(0);
    read_frags(F0, nA, nB, 0);
    issue_tile(cA, cB, min(kt + 2, KT - 1));
    mma(F1, 0);
    mma(F1, 1);
    hints_region2();
    __builtin_amdgcn_sched_barrier(0);
  };

  if (KT > 0) {
    issue_tile(sA0, sB0, 0);
    wait_vm_all();
    __syncthreads();
    read_frags(F0, sA0, sB0, 0);
    issue_tile(sA1, sB1, min(1, KT - 1));
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      step(kt, sA0, sB0, sA1, sB1);
      step(kt + 1, sA1, sB1, sA0, sB0);
    }
    if (kt < KT) step(kt, sA0, sB0, sA1, sB1);
    wait_vm_all();  // the clamped loads of the last steps
  }

  // ---- ragged last K step: masked register loads, then the same math -------
  if (k_tail) {
    __syncthreads();  // every wave is done with both stages
    const int kb = KT * BK;
    const int lrow = tid >> 3, lchk = tid & 7;
    const bool ok = kb + lchk * 8 < K;
    const int lv = (lrow * K + lchk * 8 + kb) * 2;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const u32x4 v = ok ? __builtin_amdgcn_raw_buffer_load_b128(rs_a, lv, i * 32 * K * 2, 0) : z;
      *reinterpret_cast<u32x4*>(sA0 + swz(i * 32 + lrow, lchk)) = v;
    }
#pragma unroll
    for (int i = 0; i < BN / 32; ++i) {
      u32x4 v = z;
      if (ok) {
        if constexpr (EPI == EPI_GLU) {
          v = (i < BN / 64) ? __builtin_amdgcn_raw_buffer_load_b128(rs_b0, lv, i * 32 * K * 2, 0)
                            : __builtin_amdgcn_raw_buffer_load_b128(rs_b1, lv, (i - BN / 64) * 32 * K * 2, 0);
        } else {
          v = __builtin_amdgcn_raw_buffer_load_b128(rs_b0, lv, i * 32 * K * 2, 0);
        }
      }
      *reinterpret_cast<u32x4*>(sB0 + swz(i * 32 + lrow, lchk)) = v;
    }
    __syncthreads();
    read_frags(F0, sA0, sB0, 0);
    read_frags(F1, sA0, sB0, 1);
    mma(F0, 0);
    mma(F0, 1);
    mma(F1, 0);
    mma(F1, 1);
    square(F0);
    square(F1);
  }

  // ---- deferred row scale s in the accumulator layout --------------------
  // Fragment lanes hold row (lane % 32) of subtile i; reduce over the two
  // K-chunk lane halves, publish per row through LDS, then read back in the
  // accumulator layout: element e of a lane is row 8 (e / 4) + 4 (lane / 32)
  // + e % 4, column lane % 32.
  auto acc_row = [&](int i, int e) { return wm * WM + i * 32 + 8 * (e >> 2) + 4 * fchk + (e & 3); };
  if constexpr (SUMSQ) {
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
      const int i = q * WAVES_N + wn;  // subtile this wave squared
      const float v = xor_sum<32>(ss[q]);
      if (i < TM && fchk == 0) srow_lds[wm * WM + i * 32 + frow] = rsqrtf(v * p.inv_k + p.eps);
    }
    __syncthreads();
  }
  // scales of accumulator rows acc_row(i, 4b) .. +3 (four consecutive rows)
  auto scale4 = [&](int i, int b) {
    if constexpr (SUMSQ) return *reinterpret_cast<const f32x4*>(&srow_lds[acc_row(i, 4 * b)]);
    else return f32x4{1.f, 1.f, 1.f, 1.f};
  };

  auto store = [&](int m, int n, float v) {
    if (m < M && n < N) {
      if constexpr (OUT_BF16)
        static_cast<uint16_t*>(p.Y)[(size_t)m * N + n] = (uint16_t)f32_to_bf16_bits(v);
      else
        static_cast<float*>(p.Y)[(size_t)m * N + n] = v;
    }
  };

  if constexpr (EPI == EPI_PLAIN || EPI == EPI_GLU) {
    // Output goes through LDS one accumulator row block at a time: every wave
    // writes its scaled (and gated) values for subtile row i, then the whole
    // workgroup stores the WAVES_M x 32 rows with 16-byte, line-filling
    // global stores.
    using OutT = typename std::conditional<OUT_BF16, uint16_t, float>::type;
    constexpr int OSZ = sizeof(OutT);
    constexpr int OCOLS = OUT_BN;                 // output columns of the tile
    constexpr int OLD = OCOLS + 16 / OSZ;         // padded LDS row (elements)
    constexpr int OROWS = WAVES_M * 32;           // rows per pass (32 per wave row)
    constexpr int WOUT = (EPI == EPI_GLU) ? WN / 2 : WN;  // output columns per wave
    static_assert(WAVES_M <= 2 && 32 * OLD * OSZ <= (BM + BN) * BK * 2, "a wave row's staging fits in one stage");
    // rows of wave row 0 stage in st0, of wave row 1 in st1
    auto ob_row = [&](int wrow) { return reinterpret_cast<OutT*>(wrow == 0 ? st0 : st1); };
    constexpr int CPR = OCOLS * OSZ / 16;     // 16-byte chunks per row
    const bool vec_ok = ((N * OSZ) % 16) == 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      __syncthreads();  // previous pass (or the main loop) is done with LDS
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4 sc = scale4(i, b);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = wm * 32 + 8 * b + 4 * fchk + r;
#pragma unroll
          for (int j = 0; j < ((EPI == EPI_GLU) ? TN / 2 : TN); ++j) {
            float v;
            if constexpr (EPI == EPI_GLU) {
              const float a = acc[i][j][4 * b + r] * sc[r];
              const float u = acc[i][j + TN / 2][4 * b + r] * sc[r];
              v = silu(a) * u;
            } else {
              v = acc[i][j][4 * b + r] * sc[r];
            }
            const int lc = wn * WOUT + j * 32 + frow;
            OutT* ob = ob_row(wm);
            if constexpr (OUT_BF16)
              ob[(lr - wm * 32) * OLD + lc] = (uint16_t)f32_to_bf16_bits(v);
            else
              ob[(lr - wm * 32) * OLD + lc] = v;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = tid; q < OROWS * CPR; q += kThreads) {
        const int lr = q / CPR, ch = q % CPR;
        const int wmr = lr / 32, r32 = lr % 32;
        const int m = m0 + wmr * WM + i * 32 + r32;
        const int n = n0 + ch * (16 / OSZ);
        const u32x4 v = *reinterpret_cast<const u32x4*>(&ob_row(wmr)[r32 * OLD + ch * (16 / OSZ)]);
        if (m < M) {
          if (vec_ok && n + 16 / OSZ <= N) {
            *reinterpret_cast<u32x4*>(static_cast<OutT*>(p.Y) + (size_t)m * N + n) = v;
          } else {
            const OutT* e = reinterpret_cast<const OutT*>(&v);
            for (int t = 0; t < 16 / OSZ; ++t)
              if (n + t < N) static_cast<OutT*>(p.Y)[(size_t)m * N + n + t] = e[t];
          }
        }
      }
    }
  } else {  // EPI_QKNORM
    // Head sums of C^2 per row: first over this wave's subtiles of a head
    // (registers), then over the 32 columns of a subtile (lanes), then over
    // the waves a head spans (LDS).  A head segment is the part of a head
    // inside one wave: min(head_dim, WN) columns.
    const int hd = p.head_dim;
    const int seg = hd < WN ? hd : WN;        // columns of a head segment
    const int segs_per_wave = WN / seg;       // 1, 2 or 4
    const int subs_per_seg = seg / 32;
    constexpr int SEG_SLOTS = BN / 64;        // head segments per tile row, at most
    static_assert(BM * SEG_SLOTS * 4 <= BM * BK * 2, "partials fit in one A stage");
    float* part = reinterpret_cast<float*>(st0);  // [BM][SEG_SLOTS]; stages are idle now
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        for (int sg = 0; sg < segs_per_wave; ++sg) {
          float v = 0.f;
#pragma unroll
          for (int j = 0; j < TN; ++j)
            if (j / subs_per_seg == sg) v += acc[i][j][e] * acc[i][j][e];
          v = xor_sum<1>(v);
          v = xor_sum<2>(v);
          v = xor_sum<4>(v);
          v = xor_sum<8>(v);
          v = xor_sum<16>(v);
          if (frow == 0) part[acc_row(i, e) * SEG_SLOTS + wn * segs_per_wave + sg] = v;
        }
    __syncthreads();
    const int nq_heads = p.nq_cols / hd;
    const int segs_per_head = hd / seg;  // waves a head spans
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int trow = acc_row(i, e);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int c0 = n0 + wn * WN + j * 32;  // first output column of the subtile
          const int n = c0 + frow;
          const int head = c0 / hd;  // global head index
          const int col_in_head = n - head * hd;
          float y;
          if (c0 >= p.nq_cols + p.nk_cols && p.v_mode == 0) {
            y = acc[i][j][e] * (SUMSQ ? srow_lds[trow] : 1.0f);  // v head keeps the deferred row scale
          } else {
            const int slot0 = ((wn * WN + j * 32) / hd) * segs_per_head;  // first segment of this head
            float hs = 0.f;
            for (int q = 0; q < segs_per_head; ++q) hs += part[trow * SEG_SLOTS + slot0 + q];
            float gain = 1.0f;
            if (n < N) {
              if (c0 < p.nq_cols)
                gain = p.g_q[(size_t)head * p.g_stride + col_in_head];
              else if (c0 < p.nq_cols + p.nk_cols)
                gain = p.g_k[(size_t)(head - nq_heads) * p.g_stride + col_in_head];
            }
            y = acc[i][j][e] * gain * rsqrtf(hs / (float)hd + p.eps_head);
          }
          store(m0 + trow, n, y);
        }
      }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI, bool SUMSQ, bool OUT_BF16>
hipError_t launch_cfg(const GemmArgs& a0, hipStream_t st) {
  GemmArgs a = a0;
  constexpr int OUT_BN = (EPI == EPI_GLU) ? BN / 2 : BN;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + OUT_BN - 1) / OUT_BN;
  if (a.group_m <= 0) a.group_m = 8;
  const int nblk = a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WAVES_M, WAVES_N, EPI, SUMSQ, OUT_BF16>), dim3(nblk),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int EPI, bool SUMSQ, bool OUT_BF16>
hipError_t launch_tile(int tile, const GemmArgs& a, hipStream_t st) {
  switch (tile) {
    case TILE_256x256: return launch_cfg<256, 256, 2, 2, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_128x256: return launch_cfg<128, 256, 2, 2, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_64x256:  return launch_cfg<64, 256, 1, 4, EPI, SUMSQ, OUT_BF16>(a, st);
    case TILE_128x128: return launch_cfg<128, 128, 2, 2, EPI, SUMSQ, OUT_BF16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_bf16(int epi, bool sumsq, bool out_bf16, int tile, const GemmArgs& a, hipStream_t st) {
#define FN_DISPATCH(E)                                                              \
  if (epi == E) {                                                                   \
    if (sumsq) return out_bf16 ? launch_tile<E, true, true>(tile, a, st)            \
                               : launch_tile<E, true, false>(tile, a, st);          \
    return out_bf16 ? launch_tile<E, false, true>(tile, a, st)                      \
                    : launch_tile<E, false, false>(tile, a, st);                    \
  }
  FN_DISPATCH(EPI_PLAIN)
  FN_DISPATCH(EPI_GLU)
  FN_DISPATCH(EPI_QKNORM)
#undef FN_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace fn
