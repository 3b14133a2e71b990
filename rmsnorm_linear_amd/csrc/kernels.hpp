// Internal launcher interface between the C ABI layer (api.cpp) and the
// HIP kernels.  Everything here is enqueued on the given stream; nothing
// allocates.  Argument validation happens in api.cpp before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fn {

// EPI_QKNORM_ROPE: the qknorm epilogue, then the rotary embedding of q and k.
// EPI_LN: LayerNorm deferred: y = s (z - mu c[n]) + b[n] (s = 1, mu = 0
// without the statistics: y = z + b[n]).
// EPI_LATENT: MLA attention input: latent columns [0, lat_cols) go unscaled
// to a float32 workspace with per-32-column sums of squares (a row kernel
// then applies the latent norms); the columns after them get z * s[m] and,
// with positions, the rotary embedding.
enum Epi { EPI_PLAIN = 0, EPI_GLU = 1, EPI_QKNORM = 2, EPI_QKNORM_ROPE = 3, EPI_LN = 4, EPI_LATENT = 5 };

// Prefill tiles: BM x BN with eight waves, the number of LDS stages (two
// unless named), and where the row squares come from (the MFMA x
// fragments, or "q": one pass over the LDS x tile).
enum Tile {
  TILE_256x256 = 0,
  TILE_128x256 = 1,
  TILE_64x256 = 2,
  TILE_128x128 = 3,
  TILE_128x256_S3 = 4,
  TILE_64x256_S4Q = 5,
  TILE_256x256_Q = 6,
  TILE_128x128_Q = 7,
  TILE_256x256_W3 = 8,  // plus a third stage for the weight tile
  TILE_256x256_X3 = 9,  // plus a third stage for the x tile (plain epilogue only)
  TILE_COUNT = 10
};

struct GemmArgs {
  const uint16_t* A;   // x (fused) or xn (unfused) [M x K], bf16 bits
  const uint16_t* B0;  // W* / W (plain, qknorm) or gate weight (glu) [N x K]
  const uint16_t* B1;  // up weight (glu) [N x K]
  void* Y;             // [M x N] float or bf16 bits
  int M, K, N;         // N = output columns
  float eps;           // row eps of the deferred scale
  float inv_k;         // 1 / K
  // qknorm
  const float* g_q;
  const float* g_k;
  int64_t g_stride;
  int nq_cols, nk_cols, head_dim;
  float eps_head;
  int v_mode;
  int g_vec4;  // g_q, g_k 16-byte aligned and g_stride % 4 == 0: vector gain loads
  // rotary embedding (EPI_QKNORM_ROPE)
  const int32_t* pos;   // [M] token positions
  const float* rope;    // [n_pos x rot_dim]: (cos, sin) of pair i at 2i, 2i+1
  int64_t n_pos;
  int rot_dim;          // rotated columns per head, multiple of 4, <= head_dim
  // LayerNorm (EPI_LN)
  const float* ln_c;    // [N] column sums of W* (used with the statistics)
  const float* ln_b;    // [N] output bias, or NULL
  // Row statistics from a pass before the kernel (used when the kernel does
  // not take them itself): scale s[m] and, for LayerNorm, mean mu[m].
  const float* row_s;
  const float* row_mu;
  // MLA latent (EPI_LATENT; pos / rope / n_pos / rot_dim as above, pos may be NULL)
  int lat_cols;         // latent columns, a multiple of 32
  float* lat_z;         // [M x lat_cols] float32 product of the latent columns
  float* lat_part;      // [M x lat_cols / 32] sums of squares per 32-column subtile
  // fp8 (E4M3 x and weights): channel scales of the weight (gate) and of the
  // up weight (glu); row_s then holds the row factor s[m] q_x[m]
  const float* col_q0;
  const float* col_q1;
  // filled by the launcher
  int tiles_m, tiles_n, group_m;
};

// bf16 MFMA prefill kernel.  sumsq: compute and apply the deferred row scale.
// launch_gemm_bf16_epi<E> is defined in the gemm_bf16.hip translation unit
// built for epilogue E.
template <int EPI>
hipError_t launch_gemm_bf16_epi(bool sumsq, bool out_bf16, int tile, const GemmArgs& a, hipStream_t st);
#define FN_DECLARE_GEMM_EPI(E) \
  template <>              \
  hipError_t launch_gemm_bf16_epi<E>(bool sumsq, bool out_bf16, int tile, const GemmArgs& a, hipStream_t st);
FN_DECLARE_GEMM_EPI(EPI_PLAIN)
FN_DECLARE_GEMM_EPI(EPI_GLU)
FN_DECLARE_GEMM_EPI(EPI_QKNORM)
FN_DECLARE_GEMM_EPI(EPI_QKNORM_ROPE)
FN_DECLARE_GEMM_EPI(EPI_LN)
FN_DECLARE_GEMM_EPI(EPI_LATENT)
#undef FN_DECLARE_GEMM_EPI

// The same kernel on E4M3 x and weights (A = x codes, B0 / B1 = weight
// codes, row_s = the row factors, col_q0 / col_q1 = the channel scales):
// plain and glu epilogues, defined in their translation units.
template <int EPI>
hipError_t launch_gemm_fp8_epi(bool out_bf16, int tile, const GemmArgs& a, hipStream_t st);
template <>
hipError_t launch_gemm_fp8_epi<EPI_PLAIN>(bool out_bf16, int tile, const GemmArgs& a, hipStream_t st);
template <>
hipError_t launch_gemm_fp8_epi<EPI_GLU>(bool out_bf16, int tile, const GemmArgs& a, hipStream_t st);

inline hipError_t launch_gemm_fp8(int epi, bool out_bf16, int tile, const GemmArgs& a, hipStream_t st) {
  if (epi == EPI_PLAIN) return launch_gemm_fp8_epi<EPI_PLAIN>(out_bf16, tile, a, st);
  if (epi == EPI_GLU) return launch_gemm_fp8_epi<EPI_GLU>(out_bf16, tile, a, st);
  return hipErrorInvalidValue;
}

inline hipError_t launch_gemm_bf16(int epi, bool sumsq, bool out_bf16, int tile, const GemmArgs& a, hipStream_t st) {
  switch (epi) {
    case EPI_PLAIN: return launch_gemm_bf16_epi<EPI_PLAIN>(sumsq, out_bf16, tile, a, st);
    case EPI_GLU: return launch_gemm_bf16_epi<EPI_GLU>(sumsq, out_bf16, tile, a, st);
    case EPI_QKNORM: return launch_gemm_bf16_epi<EPI_QKNORM>(sumsq, out_bf16, tile, a, st);
    case EPI_QKNORM_ROPE: return launch_gemm_bf16_epi<EPI_QKNORM_ROPE>(sumsq, out_bf16, tile, a, st);
    case EPI_LN: return launch_gemm_bf16_epi<EPI_LN>(sumsq, out_bf16, tile, a, st);
    case EPI_LATENT: return launch_gemm_bf16_epi<EPI_LATENT>(sumsq, out_bf16, tile, a, st);
  }
  return hipErrorInvalidValue;
}

struct DecodeArgs {
  const uint16_t* x;   // [M x K]
  const uint16_t* B0;  // W* or gate [N x K]
  const uint16_t* B1;  // up [N x K] (glu)
  void* Y;             // [M x N]
  int M, K, N;
  float eps, inv_k;
  const float* ln_c;   // EPI_LN: column sums of W* [N]
  const float* ln_b;   // EPI_LN: output bias [N] or NULL
  const float* q0;     // fp8 weights: channel scales of B0 [N]
  const float* q1;     // fp8 weights: channel scales of B1 [N] (glu)
  int packed;          // 0 row-major, 1 decode-packed (launch_pack_decode), 2 glu gate/up pair packed into B0
};

// Decode-packed copy of a row-major [N x row_bytes] weight (bf16 or fp8
// bytes, row_bytes a multiple of 16): ceil(N / 16) slabs of
// ceil(row_bytes / 64) steps of 64 pieces of 16 bytes.
// With W_up, the gate/up pair layout: each K step holds W's 64 pieces of
// the slab, then W_up's (twice the size).
hipError_t launch_pack_decode(const void* W, const void* W_up, int64_t N, int64_t row_bytes, void* P,
                              hipStream_t st);

// Weight-streaming kernel for M <= 16 rows (plain, glu or LayerNorm epilogue).
hipError_t launch_decode_bf16(int epi, bool sumsq, bool out_bf16, const DecodeArgs& a, hipStream_t st);

// The same kernel on E4M3 weights (B0 / B1 point to bytes, q0 / q1 the
// channel scales); plain or glu epilogue; K % 16 == 0.
hipError_t launch_decode_fp8(int epi, bool sumsq, bool out_bf16, const DecodeArgs& a, hipStream_t st);

// Per-channel E4M3 quantisation: q[n] = float32(float64(amax_n) / 448) (1 for
// a zero row), code[n,k] = RNE_E4M3(float64(W[n,k]) / q[n]), saturating.
hipError_t launch_quantize_fp8(const void* W, int w_dt, int64_t N, int64_t K, uint8_t* codes, float* q,
                               hipStream_t st);

// Rows of bf16 x [M x K] to E4M3 codes as launch_quantize_fp8 does for a
// weight (per-row scale q[m]); r[m] = q[m], or with stats s[m] q[m] where
// s[m] = 1 / sqrt(mean_k x[m,k]^2 + eps) from the same read of the row.
hipError_t launch_quantize_rows_fp8(const void* x, int64_t M, int64_t K, bool stats, float eps, uint8_t* codes,
                                    float* r, hipStream_t st);

struct GemmF32Args {
  const float* A;  // [M x K]
  const float* B;  // [N x K]
  float* Y;        // [M x N]
  int M, K, N;
  float eps, inv_k;
  const float* ln_c;  // EPI_LN: column sums of W* [N]
  const float* ln_b;  // EPI_LN: output bias [N] or NULL
};

// float32 MFMA kernel (v_mfma_f32_16x16x4_f32), plain or LayerNorm epilogue.
hipError_t launch_gemm_f32(int epi, bool sumsq, const GemmF32Args& a, hipStream_t st);

// W*[n,k] = round(g[k] * W[n,k]); dtypes 0 = f32, 1 = bf16.
hipError_t launch_fold(const void* W, int w_dt, const float* g, int64_t N, int64_t K, void* Ws, int out_dt,
                       hipStream_t st);

// LayerNorm fold: W*[n,k] = round(g[k] W[n,k]) (as launch_fold), c[n] =
// sum_k W*[n,k] over the stored values, b*[n] = sum_k beta[k] W[n,k] +
// bias[n] (beta, bias may be NULL), both sums in float64, rounded once.
hipError_t launch_fold_layernorm(const void* W, int w_dt, const float* g, const float* beta, const float* bias,
                                 int64_t N, int64_t K, void* Ws, int out_dt, float* c, float* b, hipStream_t st);

// Unfused LayerNorm baseline: xn[m,k] = round_dt((x - mu) / sqrt(var + eps) g[k] + beta[k]).
hipError_t launch_layernorm(const void* x, int dt, const float* g, const float* beta, int64_t M, int64_t K, float eps,
                            void* xn, hipStream_t st);

// Unfused baseline first kernel: xn[m,k] = round_dt(x[m,k] * s[m] * g[k]).
hipError_t launch_rmsnorm(const void* x, int dt, const float* g, int64_t M, int64_t K, float eps, void* xn,
                          hipStream_t st);

// LayerNorm row statistics: mu[m] = mean_k x[m,k], s[m] = 1 / sqrt(mean_k
// (x[m,k] - mu[m])^2 + eps), float32 vectors.
hipError_t launch_ln_stats(const void* x, int dt, int64_t M, int64_t K, float eps, float* mu, float* s,
                           hipStream_t st);

// s[m] = 1 / sqrt(mean_k x[m,k]^2 + eps) into a float32 vector.
hipError_t launch_row_scale(const void* x, int dt, int64_t M, int64_t K, float eps, float* s, hipStream_t st);

// y[m,n] = z[m,n] * s[m], z float32, y in y_dt.
hipError_t launch_post_scale(const float* z, const float* s, int64_t M, int64_t N, void* y, int y_dt,
                             hipStream_t st);

// MLA latent norms: y[m, seg] = z[m, seg] * g_seg / sqrt(mean(z[m, seg]^2) + eps)
// for the q latent [0, nq) and the kv latent [nq, lat), from the GEMM's float32
// product and 32-column sums of squares; y has row stride N, dtype y_dt.
hipError_t launch_latent_norm(const float* z, const float* part, int64_t M, int lat, int nq, const float* g_q,
                              const float* g_kv, float eps, void* y, int64_t N, int y_dt, hipStream_t st);

// Head norms of the head-norm ops at decode batch sizes, after the
// weight-streaming kernel has written z = x . W^T (no row scale, float32)
// to the workspace.  One wave per (row, head): q and k heads
// z g / sqrt(mean over the head of z^2 + eps_head), then, with pos, the
// rotary embedding at the row's position; v heads z s[m] (v_scale: s from
// the row of x), a unit-gain head norm (v_mode 1), or z as it is.
struct QkFinishArgs {
  const float* z;       // [M x N]
  const uint16_t* x;    // [M x K] bf16 (v_scale)
  int M, K, N;
  int nq_cols, nk_cols, head_dim;
  const float* g_q;
  const float* g_k;
  int64_t g_stride;
  float eps_x, eps_head, inv_k;
  int v_mode, v_scale;
  const int32_t* pos;   // NULL: no rotation
  const float* rope;
  int64_t n_pos;
  int rot_dim;
  void* y;              // [M x N]
};
hipError_t launch_qk_finish(const QkFinishArgs& a, int y_dt, hipStream_t st);

// Rotary table: t[p * rot_dim + 2i] = cos(p theta_i), t[.. + 2i + 1] =
// sin(p theta_i), theta_i = base^(-2i / rot_dim), in float64, rounded once.
hipError_t launch_rope_table(double base, int rot_dim, int64_t n_pos, float* t, hipStream_t st);

// Fill n 32-bit words with a pattern (a kernel, so it is safe under graph capture).
hipError_t launch_fill_u32(void* p, uint32_t value, int64_t n_words, hipStream_t st);

}  // namespace fn
