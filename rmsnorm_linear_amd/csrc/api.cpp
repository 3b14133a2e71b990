// C ABI of libflashnorm: argument validation, kernel selection and the
// two-stream fork/join.  Every check runs before the first launch, so a
// call that fails has enqueued nothing.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/flashnorm.h"
#include "../../include/flashnorm_testing.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(fn_status_string(status)) + ": " + buf;
  return status;
}

int ok() { return FN_OK; }

int hip_fail(hipError_t e, const char* what) {
  return fail(FN_E_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool log_on() {
  static const bool on = [] {
    const char* v = std::getenv("FN_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int kDecodeMaxRows = 16;
// Head-norm ops: the weight-streaming product plus a per-head pass beats the
// 256-column head-norm tile at every decode batch size (measured at
// K = 2560, 8 q / 4 kv heads of 256: 15.0 / 16.0 us at M = 1 / 12 against
// 24.7 us).
constexpr int kQkDecodeMaxRows = kDecodeMaxRows;

int check_dims(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 1 || N < 1) return fail(FN_E_SHAPE, "need M >= 0, K >= 1, N >= 1 (got M=%lld K=%lld N=%lld)",
                                           (long long)M, (long long)K, (long long)N);
  if (M > kMaxDim || K > kMaxDim || N > kMaxDim)
    return fail(FN_E_SHAPE, "dimension above 2^31-1");
  if (M * K > (int64_t(1) << 40) || N * K > (int64_t(1) << 40) || M * N > (int64_t(1) << 40))
    return fail(FN_E_SHAPE, "tensor above 2^40 elements");
  return FN_OK;
}

int check_dtype_triple(int x_dt, int w_dt, int y_dt) {
  if (x_dt != FN_F32 && x_dt != FN_BF16) return fail(FN_E_DTYPE, "x dtype %d", x_dt);
  if (w_dt != x_dt) return fail(FN_E_DTYPE, "weight dtype must equal x dtype");
  if (y_dt != FN_F32 && y_dt != FN_BF16) return fail(FN_E_DTYPE, "y dtype %d", y_dt);
  if (x_dt == FN_F32 && y_dt != FN_F32) return fail(FN_E_DTYPE, "f32 inputs need an f32 output");
  return FN_OK;
}

// The bf16 prefill kernel addresses a 256-row operand tile with 32-bit byte
// offsets (256 * K * 2 < 2^31).
constexpr int64_t kMaxKBf16 = int64_t(1) << 21;

int check_k_vec(int x_dt, int64_t K) {
  const int v = (x_dt == FN_BF16) ? 8 : 4;
  if (K % v) return fail(FN_E_ALIGN, "K=%lld must be a multiple of %d for this dtype", (long long)K, v);
  if (x_dt == FN_BF16 && K > kMaxKBf16)
    return fail(FN_E_UNSUPPORTED, "K=%lld above %lld is not supported for bf16", (long long)K, (long long)kMaxKBf16);
  return FN_OK;
}

int check_eps(float eps, const char* name) {
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(FN_E_ARG, "%s must be finite and >= 0", name);
  return FN_OK;
}

size_t round_up(size_t v) { return (v + 255) & ~size_t(255); }

// Row statistics in a pass of their own before the GEMM (fused variant,
// bf16; plain, LayerNorm and MLA-latent epilogues).  In the GEMM, every one
// of the N / 256 column tiles of a row block redoes the row's sums; with
// many column tiles and a large x, one pass over x is cheaper (Llama-7B
// QKV, 48 column tiles: 7.8 us against about 5% of a 340 us GEMM), and the
// GEMM without the sums has the registers for its deepest weight ring.
// With fewer column tiles the extra launch does not pay: at the MLA shape
// (2048 x 5120 -> 2112, 9 column tiles) the pass saves 2 us of kernel time
// but the step, with its gap between launches, is 3 us slower.
// FN_PRESTATS=0 / 1 forces it off / on.
bool use_prestats(int op, int64_t M, int64_t K, int64_t N, int x_dt) {
  if (x_dt != FN_BF16 || M <= kDecodeMaxRows) return false;
  if (op != FN_OP_NORM_LINEAR && op != FN_OP_LAYERNORM_LINEAR && op != FN_OP_LINEAR_LATENT_NORM) return false;
  if (const char* v = std::getenv("FN_PRESTATS")) {
    if (v[0] == '0') return false;
    if (v[0] == '1') return true;
  }
  return (N + 255) / 256 >= 16 && M * K >= (int64_t(1) << 23);
}

// Workspace of the MLA latent op: the float32 product of the latent columns
// and their 32-column sums of squares, sized for N (>= the latent width).
size_t latent_ws(int64_t M, int64_t N) {
  return ((size_t)M * N * 4 + 255) / 256 * 256 + ((size_t)M * ((N + 31) / 32) * 4 + 255) / 256 * 256;
}

bool is_fp8_op(int op) { return op == FN_OP_NORM_LINEAR_FP8 || op == FN_OP_NORM_GLU_FFN_FP8; }

// fp8 ops above decode batch sizes: x quantised per row into the workspace
// (codes, then one float32 factor per row), after the normalised x for the
// unfused baseline.
size_t fp8_prefill_ws(int variant, int64_t M, int64_t K) {
  return (variant == FN_UNFUSED ? round_up((size_t)M * (size_t)K * 2) : 0) + round_up((size_t)M * (size_t)K) +
         round_up((size_t)M * 4);
}

size_t ws_need(int op, int variant, int64_t M, int64_t K, int64_t N, int x_dt) {
  const size_t e = (x_dt == FN_BF16) ? 2 : 4;
  if (is_fp8_op(op) && M > kDecodeMaxRows) return fp8_prefill_ws(variant, M, K);
  if (op == FN_OP_LINEAR_LATENT_NORM)
    return latent_ws(M, N) + (variant == FN_UNFUSED ? round_up((size_t)M * (size_t)K * e) : 0) +
           (variant == FN_FUSED && use_prestats(op, M, K, N, x_dt) ? round_up((size_t)M * 4) : 0);
  if ((op == FN_OP_LINEAR_QKNORM || op == FN_OP_LINEAR_QKNORM_ROPE) && x_dt == FN_BF16 && M <= kQkDecodeMaxRows)
    // decode path: the weight-streaming kernel's float32 product, then the head norms
    return (variant == FN_UNFUSED ? round_up((size_t)M * (size_t)K * e) : 0) + round_up((size_t)M * (size_t)N * 4);
  if (variant == FN_UNFUSED) return round_up((size_t)M * (size_t)K * e);
  if (variant == FN_FUSED && use_prestats(op, M, K, N, x_dt))
    return round_up((size_t)M * 4) * (op == FN_OP_LAYERNORM_LINEAR ? 2 : 1);
  if (variant == FN_TWO_STREAM && op == FN_OP_NORM_LINEAR)
    return round_up((size_t)M * (size_t)N * 4) + round_up((size_t)M * 4);
  return 0;
}

int check_ws(int op, int variant, int64_t M, int64_t K, int64_t N, int x_dt, const void* ws, size_t ws_bytes) {
  const size_t need = ws_need(op, variant, M, K, N, x_dt);
  if (need == 0) return FN_OK;
  if (!ws) return fail(FN_E_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (ws_bytes < need) return fail(FN_E_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
  if (!aligned16(ws)) return fail(FN_E_ALIGN, "workspace not 16-byte aligned");
  return FN_OK;
}

// FN_FUSED_PACKED is the fused variant on decode-packed weights, offered
// where the weight-streaming kernel runs: bf16 x and M <= 16 rows.
int check_packed(int64_t M, int x_dt) {
  if (x_dt != FN_BF16) return fail(FN_E_UNSUPPORTED, "decode-packed weights take bf16 x");
  if (M > kDecodeMaxRows)
    return fail(FN_E_UNSUPPORTED, "decode-packed weights are read by the weight-streaming kernel, M <= %d",
                kDecodeMaxRows);
  return FN_OK;
}

// ---- prefill tile choice -------------------------------------------------
int pick_tile(int epi, int64_t M, int64_t N, bool sumsq) {
  if (const char* v = std::getenv("FN_TILE")) {
    const int t = std::atoi(v);
    const bool head_tiles = epi == fn::EPI_QKNORM || epi == fn::EPI_QKNORM_ROPE;  // heads within one 256-wide tile
    const bool plain_only = t == fn::TILE_256x256_X3 && epi != fn::EPI_PLAIN;
    if (t >= 0 && t < fn::TILE_COUNT && !plain_only && !(head_tiles && (t == fn::TILE_128x128 || t == fn::TILE_128x128_Q)))
      return t;
  }
  auto tiles = [&](int bm, int bn) {
    const int obn = (epi == fn::EPI_GLU) ? bn / 2 : bn;
    return ((M + bm - 1) / bm) * ((N + obn - 1) / obn);
  };
  // Three candidates, each one workgroup per CU: 256 x 256 (two stages),
  // 128 x 256 (three stages) and 64 x 256 (four stages; smaller tiles trade
  // work per K step for a deeper LDS ring).  A grid runs in ceil(tiles /
  // 256 CUs) rounds, and a K step of each tile takes, measured on the
  // prefill shapes, about 1.77 / 1.10 / 1.00 time units.  Take the least
  // rounds x step time (ties to the larger tile).
  struct Cand {
    int tile, bm;
    double t_step;
  };
  const Cand cands[3] = {{fn::TILE_256x256, 256, 1.77}, {fn::TILE_128x256_S3, 128, 1.10}, {fn::TILE_64x256_S4Q, 64, 1.00}};
  constexpr int kCUs = 256;
  int best = cands[0].tile;
  double best_cost = 1e300;
  for (const Cand& c : cands) {
    const double cost = (double)((tiles(c.bm, 256) + kCUs - 1) / kCUs) * c.t_step;
    if (cost < best_cost) {
      best_cost = cost;
      best = c.tile;
    }
  }
  // Without the squares (unfused baseline, statistics pass, two-stream
  // GEMM) the 256-row tile has the registers for a third weight stage,
  // which measured 2% faster; with them it does not.
  if (best == fn::TILE_256x256 && !sumsq) return fn::TILE_256x256_W3;
  return best;
}

// fp8 prefill tiles: 256 x 256 (two stages, rolling weight fragments) where
// it fills the chip in about a round or more, else 128 x 256 with three
// stages, else 128 x 128.
int pick_tile_f8(int epi, int64_t M, int64_t N) {
  if (const char* v = std::getenv("FN_TILE")) {
    const int t = std::atoi(v);
    if (t == fn::TILE_256x256 || t == fn::TILE_128x256 || t == fn::TILE_128x128 || t == fn::TILE_128x256_S3) return t;
  }
  const int64_t obn = epi == fn::EPI_GLU ? 128 : 256;
  const int64_t t256 = ((M + 255) / 256) * ((N + obn - 1) / obn);
  const int64_t t128 = ((M + 127) / 128) * ((N + obn - 1) / obn);
  if (epi == fn::EPI_PLAIN && t256 >= 240) return fn::TILE_256x256;  // the glu epilogue spills in that tile
  return t128 >= 192 ? fn::TILE_128x256_S3 : fn::TILE_128x128;
}

const char* tile_name(int t) {
  switch (t) {
    case fn::TILE_256x256: return "256x256";
    case fn::TILE_128x256: return "128x256";
    case fn::TILE_64x256: return "64x256";
    case fn::TILE_128x128: return "128x128";
    case fn::TILE_128x256_S3: return "128x256s3";
    case fn::TILE_64x256_S4Q: return "64x256s4q";
    case fn::TILE_256x256_Q: return "256x256q";
    case fn::TILE_128x128_Q: return "128x128q";
    case fn::TILE_256x256_W3: return "256x256w3";
    case fn::TILE_256x256_X3: return "256x256x3";
  }
  return "?";
}

const char* epi_name(int e) {
  switch (e) {
    case fn::EPI_PLAIN: return "plain";
    case fn::EPI_GLU: return "glu";
    case fn::EPI_QKNORM: return "qknorm";
    case fn::EPI_QKNORM_ROPE: return "qknorm_rope";
    case fn::EPI_LN: return "layernorm";
    case fn::EPI_LATENT: return "latent";
  }
  return "?";
}

int epi_of_op(int op) {
  switch (op) {
    case FN_OP_NORM_LINEAR: return fn::EPI_PLAIN;
    case FN_OP_NORM_GLU_FFN: return fn::EPI_GLU;
    case FN_OP_NORM_LINEAR_FP8: return fn::EPI_PLAIN;
    case FN_OP_NORM_GLU_FFN_FP8: return fn::EPI_GLU;
    case FN_OP_LINEAR_LATENT_NORM: return fn::EPI_LATENT;
    case FN_OP_LINEAR_QKNORM: return fn::EPI_QKNORM;
    case FN_OP_LINEAR_QKNORM_ROPE: return fn::EPI_QKNORM_ROPE;
  }
  return fn::EPI_LN;
}

// Epilogues the weight-streaming decode kernel has (the head-norm ones
// stay on the prefill kernel at every M).
bool decode_epi(int e) { return e == fn::EPI_PLAIN || e == fn::EPI_GLU || e == fn::EPI_LN; }


std::string describe(int epi, int variant, int64_t M, int64_t K, int64_t N, int x_dt, int y_dt) {
  char buf[160];
  const char* out = y_dt == FN_BF16 ? "bf16" : "f32";
  const char* var = variant == FN_FUSED          ? "fused"
                    : variant == FN_UNFUSED      ? "unfused"
                    : variant == FN_FUSED_PACKED ? "fused_packed"
                                                 : "two_stream";
  const char* pre = variant != FN_UNFUSED ? "" : epi == fn::EPI_LN ? "layernorm+" : "rmsnorm+";
  if (x_dt == FN_F32) {
    snprintf(buf, sizeof(buf), "%s:%sgemm_f32<16x32,%s>", var, pre, epi_name(epi));
  } else if (variant == FN_TWO_STREAM) {
    snprintf(buf, sizeof(buf), "%s:gemm_bf16<%s,z=f32>+row_scale+post_scale<%s>", var,
             tile_name(pick_tile(fn::EPI_PLAIN, M, N, false)), out);
  } else if (M <= kDecodeMaxRows && decode_epi(epi)) {
    snprintf(buf, sizeof(buf), "%s:%sdecode_bf16<%s,%s>", var, pre, epi_name(epi), out);
  } else if (M <= kQkDecodeMaxRows && (epi == fn::EPI_QKNORM || epi == fn::EPI_QKNORM_ROPE)) {
    snprintf(buf, sizeof(buf), "%s:%sdecode_bf16<plain,f32>+qk_finish<%s,%s>", var, pre, epi_name(epi), out);
  } else if (variant == FN_FUSED &&
             use_prestats(epi == fn::EPI_LN       ? FN_OP_LAYERNORM_LINEAR
                          : epi == fn::EPI_PLAIN  ? FN_OP_NORM_LINEAR
                          : epi == fn::EPI_LATENT ? FN_OP_LINEAR_LATENT_NORM
                                                  : -1,
                          M, K, N, x_dt)) {
    snprintf(buf, sizeof(buf), "%s:%s+gemm_bf16<%s,%s,%s>%s", var, epi == fn::EPI_LN ? "ln_stats" : "row_scale",
             tile_name(pick_tile(epi, M, N, false)), epi_name(epi), out,
             epi == fn::EPI_LATENT ? "+latent_norm" : "");
  } else {
    snprintf(buf, sizeof(buf), "%s:%sgemm_bf16<%s,%s,%s>%s", var, pre,
             tile_name(pick_tile(epi, M, N, variant == FN_FUSED)), epi_name(epi), out,
             epi == fn::EPI_LATENT ? "+latent_norm" : "");
  }
  return buf;
}

// ---- per-thread events of the two-stream variant ---------------------------
struct Events {
  hipEvent_t fork = nullptr, gemm_done = nullptr;
  ~Events() { release(); }
  void release() {
    if (fork) (void)hipEventDestroy(fork);
    if (gemm_done) (void)hipEventDestroy(gemm_done);
    fork = gemm_done = nullptr;
  }
  hipError_t ensure() {
    hipError_t e = hipSuccess;
    if (!fork) e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess && !gemm_done) e = hipEventCreateWithFlags(&gemm_done, hipEventDisableTiming);
    return e;
  }
};
thread_local Events g_events;

// Test-only: the calling thread's two-stream calls leave out the join
// (fn_testing_skip_join).  Off unless a test turns it on.
thread_local bool g_skip_join = false;

// Test-only: event pairs recorded around the calling thread's prefill GEMM
// launches (fn_testing_gemm_events), so a measurement harness can time the
// GEMM of a step that launches a pass before or after it.  Off (n == 0)
// unless the harness sets it.
struct GemmTiming {
  void* const* starts = nullptr;
  void* const* stops = nullptr;
  int n = 0;
  int i = 0;
};
thread_local GemmTiming g_gemm_timing;

// launch() (returning hipError_t), between the timing events when they are set
template <class F>
hipError_t timed_gemm(hipStream_t st, F launch) {
  GemmTiming& t = g_gemm_timing;
  if (t.n <= 0) return launch();
  const int k = t.i++ % t.n;
  hipError_t e = hipEventRecord(static_cast<hipEvent_t>(t.starts[k]), st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  return hipEventRecord(static_cast<hipEvent_t>(t.stops[k]), st);
}

// Launch the bf16 prefill/decode kernels for one op after validation.
int run_bf16(int epi, bool fused, const void* xin, const void* B0, const void* B1, int64_t M, int64_t K, int64_t N,
             float eps, void* y, int y_dt, const fn::GemmArgs* qk, hipStream_t st, int packed = 0) {
  const bool out_bf16 = y_dt == FN_BF16;
  hipError_t e;
  if (M <= kDecodeMaxRows && decode_epi(epi)) {
    fn::DecodeArgs d{};
    d.x = static_cast<const uint16_t*>(xin);
    d.B0 = static_cast<const uint16_t*>(B0);
    d.B1 = static_cast<const uint16_t*>(B1);
    d.Y = y;
    d.M = (int)M; d.K = (int)K; d.N = (int)N;
    d.eps = eps; d.inv_k = 1.0f / (float)K;
    d.packed = packed;
    if (qk) {
      d.ln_c = qk->ln_c;
      d.ln_b = qk->ln_b;
    }
    e = fn::launch_decode_bf16(epi, fused, out_bf16, d, st);
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    return ok();
  }
  fn::GemmArgs a{};
  if (qk) a = *qk;
  a.A = static_cast<const uint16_t*>(xin);
  a.B0 = static_cast<const uint16_t*>(B0);
  a.B1 = static_cast<const uint16_t*>(B1);
  a.Y = y;
  a.M = (int)M; a.K = (int)K; a.N = (int)N;
  a.eps = eps; a.inv_k = 1.0f / (float)K;
  if (const char* g = std::getenv("FN_GROUP_M")) a.group_m = std::atoi(g);
  e = timed_gemm(st, [&] { return fn::launch_gemm_bf16(epi, fused, out_bf16, pick_tile(epi, M, N, fused), a, st); });
  if (e != hipSuccess) return hip_fail(e, "gemm kernel launch");
  return ok();
}

// fn_linear_qknorm and fn_linear_qknorm_rope (rope != NULL carries the
// rotary arguments, already validated).
int qknorm_impl(const void* x, int x_dtype, int64_t M, int64_t K, const void* W_qkv, int w_dtype, int n_q_heads,
                int n_kv_heads, int head_dim, const float* g_q, const float* g_k, int64_t g_head_stride, float eps_x,
                float eps_head, int v_mode, const fn::GemmArgs* rope, const float* g1, void* y, int y_dtype,
                int variant, void* ws, size_t ws_bytes, void* stream) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(FN_E_SHAPE, "head_dim must be 64, 128 or 256 (got %d)", head_dim);
  if (n_q_heads < 1 || n_kv_heads < 1) return fail(FN_E_SHAPE, "need n_q_heads >= 1 and n_kv_heads >= 1");
  const int64_t N = (int64_t)(n_q_heads + 2 * (int64_t)n_kv_heads) * head_dim;
  if (int s = check_dims(M, K, N)) return s;
  if (int s = check_dtype_triple(x_dtype, w_dtype, y_dtype)) return s;
  if (variant != FN_FUSED && variant != FN_UNFUSED) {
    if (variant == FN_FUSED_PACKED) return fail(FN_E_UNSUPPORTED, "decode-packed weights: plain, glu or LayerNorm ops only");
    if (variant == FN_TWO_STREAM) return fail(FN_E_UNSUPPORTED, "the two-stream variant is offered for fn_norm_linear only");
    return fail(FN_E_ARG, "variant %d", variant);
  }
  if (v_mode != 0 && v_mode != 1) return fail(FN_E_ARG, "v_mode must be 0 or 1");
  if (g_head_stride < 0) return fail(FN_E_ARG, "g_head_stride must be >= 0");
  if (g_head_stride > 0 && g_head_stride < head_dim) return fail(FN_E_ARG, "g_head_stride must be 0 or >= head_dim");
  if (!W_qkv || !g_q || !g_k || (M > 0 && (!x || !y)))
    return fail(FN_E_NULL, "W_qkv, g_q and g_k are required, and x and y when M > 0");
  if (!aligned16(x) || !aligned16(W_qkv) || !aligned16(y) || (g1 && !aligned16(g1)))
    return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (int s = check_k_vec(x_dtype, K)) return s;
  if (int s = check_eps(eps_x, "eps_x")) return s;
  if (int s = check_eps(eps_head, "eps_head")) return s;
  if (variant == FN_UNFUSED && !g1) return fail(FN_E_NULL, "the unfused variant needs the first norm's gain g1");
  if (variant == FN_FUSED && g1) return fail(FN_E_ARG, "the fused variant takes the folded W_qkv; g1 must be NULL");
  if (x_dtype != FN_BF16) return fail(FN_E_UNSUPPORTED, "the qknorm ops are bf16 only");
  if (int s = check_ws(FN_OP_LINEAR_QKNORM, variant, M, K, N, x_dtype, ws, ws_bytes)) return s;
  if (M == 0) return ok();
  const int epi = rope ? fn::EPI_QKNORM_ROPE : fn::EPI_QKNORM;
  if (log_on())
    fprintf(stderr, "[flashnorm] linear_%s M=%lld K=%lld N=%lld -> %s\n", epi_name(epi), (long long)M, (long long)K,
            (long long)N, describe(epi, variant, M, K, N, x_dtype, y_dtype).c_str());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const void* xin = x;
  if (variant == FN_UNFUSED) {
    hipError_t e = fn::launch_rmsnorm(x, 1, g1, M, K, eps_x, ws, st);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
    xin = ws;
  }
  fn::GemmArgs qk{};
  if (rope) qk = *rope;
  qk.g_q = g_q;
  qk.g_k = g_k;
  qk.g_stride = g_head_stride;
  qk.g_vec4 = aligned16(g_q) && aligned16(g_k) && (g_head_stride % 4) == 0;
  qk.nq_cols = n_q_heads * head_dim;
  qk.nk_cols = n_kv_heads * head_dim;
  qk.head_dim = head_dim;
  qk.eps_head = eps_head;
  qk.v_mode = variant == FN_FUSED ? v_mode : (v_mode == 1 ? 1 : 0);
  if (M <= kQkDecodeMaxRows) {
    // Decode batch sizes: a head-norm tile would leave most of the chip
    // idle, so the weight-streaming kernel writes z = x . W^T (float32, no
    // row scale) to the workspace and a second kernel applies the head
    // norms (and the rotation) per (row, head).
    float* z = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                        (variant == FN_UNFUSED ? round_up((size_t)M * (size_t)K * 2) : 0));
    fn::DecodeArgs d{};
    d.x = static_cast<const uint16_t*>(xin);
    d.B0 = static_cast<const uint16_t*>(W_qkv);
    d.Y = z;
    d.M = (int)M; d.K = (int)K; d.N = (int)N;
    d.eps = eps_x; d.inv_k = 1.0f / (float)K;
    hipError_t e = fn::launch_decode_bf16(fn::EPI_PLAIN, false, false, d, st);
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    fn::QkFinishArgs f{};
    f.z = z;
    f.x = static_cast<const uint16_t*>(x);
    f.M = (int)M; f.K = (int)K; f.N = (int)N;
    f.nq_cols = qk.nq_cols; f.nk_cols = qk.nk_cols; f.head_dim = head_dim;
    f.g_q = g_q; f.g_k = g_k; f.g_stride = g_head_stride;
    f.eps_x = eps_x; f.eps_head = eps_head; f.inv_k = 1.0f / (float)K;
    f.v_mode = qk.v_mode;
    f.v_scale = variant == FN_FUSED && v_mode == 0;  // the unfused input is already normalised
    if (rope) {
      f.pos = rope->pos; f.rope = rope->rope; f.n_pos = rope->n_pos; f.rot_dim = rope->rot_dim;
    }
    f.y = y;
    e = fn::launch_qk_finish(f, y_dtype == FN_BF16 ? 1 : 0, st);
    if (e != hipSuccess) return hip_fail(e, "qk_finish kernel launch");
    return ok();
  }
  return run_bf16(epi, variant == FN_FUSED, xin, W_qkv, nullptr, M, K, N, eps_x, y, y_dtype, &qk, st);
}

// fn_norm_linear_fp8 / fn_norm_glu_ffn_fp8 (B1 / q1 NULL for the former).
int fp8_impl(int op, const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* B0, const float* q0,
             const uint8_t* B1, const float* q1, int64_t N, const float* g, float eps, void* y, int y_dtype,
             int variant, void* ws, size_t ws_bytes, void* stream) {
  if (int s = check_dims(M, K, N)) return s;
  if (x_dtype != FN_BF16) return fail(FN_E_DTYPE, "fp8-weight ops take bf16 x");
  if (y_dtype != FN_F32 && y_dtype != FN_BF16) return fail(FN_E_DTYPE, "y dtype %d", y_dtype);
  const bool packed = variant == FN_FUSED_PACKED;
  if (packed) {
    if (int s = check_packed(M, x_dtype)) return s;
    variant = FN_FUSED;
  }
  if (variant != FN_FUSED && variant != FN_UNFUSED) {
    if (variant == FN_TWO_STREAM) return fail(FN_E_UNSUPPORTED, "the two-stream variant is offered for fn_norm_linear only");
    return fail(FN_E_ARG, "variant %d", variant);
  }
  if (!B0 || !q0 || (M > 0 && (!x || !y)))
    return fail(FN_E_NULL, "the fp8 weights and their scales are required, and x and y when M > 0");
  for (const void* q : {(const void*)x, (const void*)B0, (const void*)q0, (const void*)B1, (const void*)q1,
                        (const void*)y, (const void*)g})
    if (q && !aligned16(q)) return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (K % 16) return fail(FN_E_ALIGN, "K=%lld must be a multiple of 16 for fp8 weights", (long long)K);
  if (int s = check_eps(eps, "eps")) return s;
  if (variant == FN_UNFUSED && !g) return fail(FN_E_NULL, "the unfused variant needs the gain g");
  if (variant == FN_FUSED && g) return fail(FN_E_ARG, "the fused variant takes the quantised folded weight; g must be NULL");
  if (M > kDecodeMaxRows && K > kMaxKBf16)
    return fail(FN_E_UNSUPPORTED, "K=%lld above %lld is not supported", (long long)K, (long long)kMaxKBf16);
  if (int s = check_ws(op, variant, M, K, N, x_dtype, ws, ws_bytes)) return s;
  if (M == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int epi = op == FN_OP_NORM_GLU_FFN_FP8 ? fn::EPI_GLU : fn::EPI_PLAIN;
  if (M > kDecodeMaxRows) {
    // Prefill: x (or, unfused, the normalised x) quantised per row to E4M3,
    // the row factor s q_x (q_x alone when unfused) from the same read; then
    // the fp8 product with the factor and the channel scales in its epilogue.
    if (log_on())
      fprintf(stderr, "[flashnorm] fp8 op M=%lld K=%lld N=%lld -> %s quant_rows+gemm_fp8<%s>\n", (long long)M,
              (long long)K, (long long)N, variant == FN_FUSED ? "fused" : "unfused",
              tile_name(pick_tile_f8(epi, M, N)));
    char* w = static_cast<char*>(ws);
    const void* xin = x;
    hipError_t e;
    if (variant == FN_UNFUSED) {
      e = fn::launch_rmsnorm(x, 1, g, M, K, eps, w, st);
      if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
      xin = w;
      w += round_up((size_t)M * (size_t)K * 2);
    }
    uint8_t* xq = reinterpret_cast<uint8_t*>(w);
    float* r = reinterpret_cast<float*>(w + round_up((size_t)M * (size_t)K));
    e = fn::launch_quantize_rows_fp8(xin, M, K, variant == FN_FUSED, eps, xq, r, st);
    if (e != hipSuccess) return hip_fail(e, "quantize_rows kernel launch");
    fn::GemmArgs a{};
    a.A = reinterpret_cast<const uint16_t*>(xq);
    a.B0 = reinterpret_cast<const uint16_t*>(B0);
    a.B1 = reinterpret_cast<const uint16_t*>(B1);
    a.Y = y;
    a.M = (int)M; a.K = (int)K; a.N = (int)N;
    a.eps = eps; a.inv_k = 1.0f / (float)K;
    a.row_s = r;
    a.col_q0 = q0;
    a.col_q1 = q1;
    if (const char* gm = std::getenv("FN_GROUP_M")) a.group_m = std::atoi(gm);
    e = timed_gemm(st, [&] { return fn::launch_gemm_fp8(epi, y_dtype == FN_BF16, pick_tile_f8(epi, M, N), a, st); });
    if (e != hipSuccess) return hip_fail(e, "gemm_fp8 kernel launch");
    return ok();
  }
  const void* xin = x;
  if (variant == FN_UNFUSED) {
    hipError_t e = fn::launch_rmsnorm(x, 1, g, M, K, eps, ws, st);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
    xin = ws;
  }
  fn::DecodeArgs d{};
  d.x = static_cast<const uint16_t*>(xin);
  d.B0 = reinterpret_cast<const uint16_t*>(B0);
  d.B1 = reinterpret_cast<const uint16_t*>(B1);
  d.q0 = q0;
  d.q1 = q1;
  d.packed = !packed ? 0 : (op == FN_OP_NORM_GLU_FFN_FP8 && B1 == nullptr) ? 2 : 1;
  d.Y = y;
  d.M = (int)M; d.K = (int)K; d.N = (int)N;
  d.eps = eps; d.inv_k = 1.0f / (float)K;
  hipError_t e = fn::launch_decode_fp8(op == FN_OP_NORM_GLU_FFN_FP8 ? fn::EPI_GLU : fn::EPI_PLAIN,
                                       variant == FN_FUSED, y_dtype == FN_BF16, d, st);
  if (e != hipSuccess) return hip_fail(e, "decode_fp8 kernel launch");
  return ok();
}

}  // namespace

// ---- the library's own scratch for fn_norm_linear_noalloc -----------------
// One array per GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in: its device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
namespace {
constexpr size_t kScratchBytes = size_t(4) << 20;  // row statistics of up to 2^20 rows
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's scratch (taken on the first call made on
// the device), or nullptr with the HIP error in *err.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int fn_abi_version(void) { return FN_ABI_VERSION; }

const char* fn_last_error(void) { return g_last_error.c_str(); }

const char* fn_status_string(int s) {
  switch (s) {
    case FN_OK: return "FN_OK";
    case FN_E_NULL: return "FN_E_NULL";
    case FN_E_SHAPE: return "FN_E_SHAPE";
    case FN_E_DTYPE: return "FN_E_DTYPE";
    case FN_E_ALIGN: return "FN_E_ALIGN";
    case FN_E_WORKSPACE: return "FN_E_WORKSPACE";
    case FN_E_UNSUPPORTED: return "FN_E_UNSUPPORTED";
    case FN_E_HIP: return "FN_E_HIP";
    case FN_E_ARG: return "FN_E_ARG";
  }
  return "FN_E_UNKNOWN";
}

int fn_workspace_bytes(int op, int variant, int64_t M, int64_t K, int64_t N, int x_dtype, size_t* out_bytes) {
  if (!out_bytes) return fail(FN_E_NULL, "out_bytes is NULL");
  if (op < FN_OP_NORM_LINEAR || op > FN_OP_LINEAR_LATENT_NORM) return fail(FN_E_ARG, "op %d", op);
  if (variant < FN_FUSED || variant > FN_FUSED_PACKED) return fail(FN_E_ARG, "variant %d", variant);
  if (x_dtype != FN_F32 && x_dtype != FN_BF16) return fail(FN_E_DTYPE, "x dtype %d", x_dtype);
  if (int s = check_dims(M, K, N)) return s;
  *out_bytes = variant == FN_FUSED_PACKED ? 0 : ws_need(op, variant, M, K, N, x_dtype);
  return ok();
}

int fn_dispatch_name(int op, int variant, int64_t M, int64_t K, int64_t N, int x_dtype, int y_dtype, char* buf,
                     size_t len) {
  if (!buf || len == 0) return fail(FN_E_NULL, "buf is NULL or empty");
  if (op < FN_OP_NORM_LINEAR || op > FN_OP_LINEAR_LATENT_NORM) return fail(FN_E_ARG, "op %d", op);
  if (variant < FN_FUSED || variant > FN_FUSED_PACKED) return fail(FN_E_ARG, "variant %d", variant);
  if (int s = check_dims(M, K, N)) return s;
  const int epi = epi_of_op(op);
  if (variant == FN_FUSED_PACKED) {
    if (!decode_epi(epi)) return fail(FN_E_UNSUPPORTED, "decode-packed weights: plain, glu or LayerNorm ops only");
    if (int s = check_packed(M, x_dtype)) return s;
  }
  if ((op == FN_OP_NORM_LINEAR_FP8 || op == FN_OP_NORM_GLU_FFN_FP8) && M > kDecodeMaxRows) {
    if (variant == FN_FUSED_PACKED) return fail(FN_E_UNSUPPORTED, "decode-packed weights take M <= %d", kDecodeMaxRows);
    snprintf(buf, len, "%s:%squant_rows+gemm_fp8<%s,%s,%s>", variant == FN_FUSED ? "fused" : "unfused",
             variant == FN_UNFUSED ? "rmsnorm+" : "", tile_name(pick_tile_f8(epi, M, N)), epi_name(epi),
             y_dtype == FN_BF16 ? "bf16" : "f32");
    return ok();
  }
  if (op == FN_OP_NORM_LINEAR_FP8 || op == FN_OP_NORM_GLU_FFN_FP8) {
    snprintf(buf, len, "%s:%sdecode_fp8<%s,%s>",
             variant == FN_FUSED ? "fused" : variant == FN_FUSED_PACKED ? "fused_packed" : "unfused",
             variant == FN_UNFUSED ? "rmsnorm+" : "", epi_name(epi), y_dtype == FN_BF16 ? "bf16" : "f32");
    return ok();
  }
  const std::string d = describe(epi, variant, M, K, N, x_dtype, y_dtype);
  snprintf(buf, len, "%s", d.c_str());
  return ok();
}

int fn_fold_weights(const void* W, int w_dtype, const float* g, int64_t N, int64_t K, void* W_star, int out_dtype,
                    void* stream) {
  if (N < 0 || K < 0) return fail(FN_E_SHAPE, "N and K must be >= 0");
  if (N > kMaxDim || K > kMaxDim || N * K > (int64_t(1) << 40)) return fail(FN_E_SHAPE, "weight too large");
  if ((w_dtype != FN_F32 && w_dtype != FN_BF16) || (out_dtype != FN_F32 && out_dtype != FN_BF16))
    return fail(FN_E_DTYPE, "dtypes must be FN_F32 or FN_BF16");
  if (N == 0 || K == 0) return ok();
  if (!W || !g || !W_star) return fail(FN_E_NULL, "W, g and W_star are required");
  if (!aligned16(W) || !aligned16(g) || !aligned16(W_star)) return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  const int vec = (w_dtype == FN_BF16 || out_dtype == FN_BF16) ? 8 : 4;
  if (K % vec) return fail(FN_E_ALIGN, "K=%lld must be a multiple of %d", (long long)K, vec);
  const size_t in_b = (size_t)N * K * (w_dtype == FN_BF16 ? 2 : 4);
  const size_t out_b = (size_t)N * K * (out_dtype == FN_BF16 ? 2 : 4);
  const uintptr_t a0 = (uintptr_t)W, a1 = a0 + in_b, b0 = (uintptr_t)W_star, b1 = b0 + out_b;
  const bool overlap = a0 < b1 && b0 < a1;
  if (overlap && !(a0 == b0 && w_dtype == out_dtype))
    return fail(FN_E_ARG, "W_star may alias W only exactly and with equal dtypes");
  hipError_t e = fn::launch_fold(W, w_dtype, g, N, K, W_star, out_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fold kernel launch");
  return ok();
}

int fn_norm_linear(const void* x, int x_dtype, int64_t M, int64_t K, const void* W, int w_dtype, int64_t N,
                   const float* g, float eps, void* y, int y_dtype, int variant, void* ws, size_t ws_bytes,
                   void* stream, void* stream_aux) {
  if (int s = check_dims(M, K, N)) return s;
  if (int s = check_dtype_triple(x_dtype, w_dtype, y_dtype)) return s;
  if (variant < FN_FUSED || variant > FN_FUSED_PACKED) return fail(FN_E_ARG, "variant %d", variant);
  const bool packed = variant == FN_FUSED_PACKED;
  if (packed) {
    if (int s = check_packed(M, x_dtype)) return s;
    variant = FN_FUSED;
  }
  if (!W || (M > 0 && (!x || !y))) return fail(FN_E_NULL, "W is required, and x and y when M > 0");
  if (!aligned16(x) || !aligned16(W) || !aligned16(y) || (g && !aligned16(g)))
    return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (int s = check_k_vec(x_dtype, K)) return s;
  if (int s = check_eps(eps, "eps")) return s;
  if (variant == FN_UNFUSED && !g) return fail(FN_E_NULL, "the unfused variant needs the gain g");
  if (variant != FN_UNFUSED && g) return fail(FN_E_ARG, "fused variants take the folded W*; g must be NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStream_t aux = static_cast<hipStream_t>(stream_aux);
  if (variant == FN_TWO_STREAM) {
    if (!aux) return fail(FN_E_NULL, "the two-stream variant needs stream_aux");
    if (aux == st) return fail(FN_E_ARG, "stream_aux must differ from stream");
    if (N % 4) return fail(FN_E_SHAPE, "the two-stream variant needs N %% 4 == 0");
    if (x_dtype != FN_BF16) return fail(FN_E_UNSUPPORTED, "the two-stream variant is bf16 only");
  }
  if (int s = check_ws(FN_OP_NORM_LINEAR, variant, M, K, N, x_dtype, ws, ws_bytes)) return s;
  if (M == 0) return ok();
  if (log_on())
    fprintf(stderr, "[flashnorm] norm_linear M=%lld K=%lld N=%lld -> %s\n", (long long)M, (long long)K,
            (long long)N, describe(fn::EPI_PLAIN, variant, M, K, N, x_dtype, y_dtype).c_str());

  hipError_t e;
  if (x_dtype == FN_F32) {
    const float* xin = static_cast<const float*>(x);
    if (variant == FN_UNFUSED) {
      e = fn::launch_rmsnorm(x, 0, g, M, K, eps, ws, st);
      if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
      xin = static_cast<const float*>(ws);
    }
    fn::GemmF32Args a{xin, static_cast<const float*>(W), static_cast<float*>(y), (int)M, (int)K, (int)N, eps,
                      1.0f / (float)K};
    e = fn::launch_gemm_f32(fn::EPI_PLAIN, variant == FN_FUSED, a, st);
    if (e != hipSuccess) return hip_fail(e, "gemm_f32 kernel launch");
    return ok();
  }

  if (variant == FN_FUSED) {
    if (use_prestats(FN_OP_NORM_LINEAR, M, K, N, x_dtype)) {
      float* srow = static_cast<float*>(ws);
      e = fn::launch_row_scale(x, 1, M, K, eps, srow, st);
      if (e != hipSuccess) return hip_fail(e, "row_scale kernel launch");
      fn::GemmArgs pre{};
      pre.row_s = srow;
      return run_bf16(fn::EPI_PLAIN, false, x, W, nullptr, M, K, N, eps, y, y_dtype, &pre, st);
    }
    return run_bf16(fn::EPI_PLAIN, true, x, W, nullptr, M, K, N, eps, y, y_dtype, nullptr, st, packed);
  }
  if (variant == FN_UNFUSED) {
    e = fn::launch_rmsnorm(x, 1, g, M, K, eps, ws, st);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
    return run_bf16(fn::EPI_PLAIN, false, ws, W, nullptr, M, K, N, eps, y, y_dtype, nullptr, st);
  }

  // FN_TWO_STREAM: fork -> {aux: GEMM into z; main: row scale into s} -> join -> post-scale
  if ((e = g_events.ensure()) != hipSuccess) return hip_fail(e, "hipEventCreate");
  float* z = static_cast<float*>(ws);
  float* srow = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up((size_t)M * N * 4));
  if ((e = hipEventRecord(g_events.fork, st)) != hipSuccess) return hip_fail(e, "hipEventRecord(fork)");
  if ((e = hipStreamWaitEvent(aux, g_events.fork, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(fork)");
  fn::GemmArgs a{};
  a.A = static_cast<const uint16_t*>(x);
  a.B0 = static_cast<const uint16_t*>(W);
  a.Y = z;
  a.M = (int)M; a.K = (int)K; a.N = (int)N;
  a.eps = eps; a.inv_k = 1.0f / (float)K;
  e = fn::launch_gemm_bf16(fn::EPI_PLAIN, false, false, pick_tile(fn::EPI_PLAIN, M, N, false), a, aux);
  if (e != hipSuccess) return hip_fail(e, "gemm kernel launch (aux stream)");
  if ((e = hipEventRecord(g_events.gemm_done, aux)) != hipSuccess) return hip_fail(e, "hipEventRecord(gemm_done)");
  e = fn::launch_row_scale(x, 1, M, K, eps, srow, st);
  if (e != hipSuccess) return hip_fail(e, "row_scale kernel launch");
  // the explicit join: the post-scale must not start before the GEMM ends
  if (!g_skip_join) {
    if ((e = hipStreamWaitEvent(st, g_events.gemm_done, 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent(join)");
  }
  e = fn::launch_post_scale(z, srow, M, N, y, y_dtype, st);
  if (e != hipSuccess) return hip_fail(e, "post_scale kernel launch");
  return ok();
}

int fn_norm_glu_ffn(const void* x, int x_dtype, int64_t M, int64_t K, const void* W_gate, const void* W_up,
                    int w_dtype, int64_t N, const float* g, float eps, void* h, int h_dtype, int variant, void* ws,
                    size_t ws_bytes, void* stream) {
  if (int s = check_dims(M, K, N)) return s;
  if (int s = check_dtype_triple(x_dtype, w_dtype, h_dtype)) return s;
  const bool packed = variant == FN_FUSED_PACKED;
  if (packed) {
    if (int s = check_packed(M, x_dtype)) return s;
    variant = FN_FUSED;
  }
  if (variant != FN_FUSED && variant != FN_UNFUSED) {
    if (variant == FN_TWO_STREAM) return fail(FN_E_UNSUPPORTED, "the two-stream variant is offered for fn_norm_linear only");
    return fail(FN_E_ARG, "variant %d", variant);
  }
  if (!W_gate || (!W_up && !packed) || (M > 0 && (!x || !h)))
    return fail(FN_E_NULL, "W_gate and W_up are required (W_up NULL only with a packed gate/up pair), and x and h when M > 0");
  if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(h) || (g && !aligned16(g)))
    return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (int s = check_k_vec(x_dtype, K)) return s;
  if (int s = check_eps(eps, "eps")) return s;
  if (variant == FN_UNFUSED && !g) return fail(FN_E_NULL, "the unfused variant needs the gain g");
  if (variant == FN_FUSED && g) return fail(FN_E_ARG, "the fused variant takes folded weights; g must be NULL");
  if (x_dtype != FN_BF16) return fail(FN_E_UNSUPPORTED, "fn_norm_glu_ffn is bf16 only");
  if (int s = check_ws(FN_OP_NORM_GLU_FFN, variant, M, K, N, x_dtype, ws, ws_bytes)) return s;
  if (M == 0) return ok();
  if (log_on())
    fprintf(stderr, "[flashnorm] norm_glu_ffn M=%lld K=%lld N=%lld -> %s\n", (long long)M, (long long)K,
            (long long)N, describe(fn::EPI_GLU, variant, M, K, N, x_dtype, h_dtype).c_str());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const void* xin = x;
  if (variant == FN_UNFUSED) {
    hipError_t e = fn::launch_rmsnorm(x, 1, g, M, K, eps, ws, st);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
    xin = ws;
  }
  return run_bf16(fn::EPI_GLU, variant == FN_FUSED, xin, W_gate, W_up, M, K, N, eps, h, h_dtype, nullptr, st,
                  packed ? (W_up ? 1 : 2) : 0);
}

int fn_linear_qknorm(const void* x, int x_dtype, int64_t M, int64_t K, const void* W_qkv, int w_dtype,
                     int n_q_heads, int n_kv_heads, int head_dim, const float* g_q, const float* g_k,
                     int64_t g_head_stride, float eps_x, float eps_head, int v_mode, const float* g1, void* y,
                     int y_dtype, int variant, void* ws, size_t ws_bytes, void* stream) {
  return qknorm_impl(x, x_dtype, M, K, W_qkv, w_dtype, n_q_heads, n_kv_heads, head_dim, g_q, g_k, g_head_stride,
                     eps_x, eps_head, v_mode, nullptr, g1, y, y_dtype, variant, ws, ws_bytes, stream);
}

int fn_linear_qknorm_rope(const void* x, int x_dtype, int64_t M, int64_t K, const void* W_qkv, int w_dtype,
                          int n_q_heads, int n_kv_heads, int head_dim, const float* g_q, const float* g_k,
                          int64_t g_head_stride, float eps_x, float eps_head, int v_mode, const int32_t* positions,
                          const float* rope_table, int64_t n_pos, int rot_dim, const float* g1, void* y,
                          int y_dtype, int variant, void* ws, size_t ws_bytes, void* stream) {
  if (!rope_table || (M > 0 && !positions))
    return fail(FN_E_NULL, "rope_table is required, and positions when M > 0");
  if (!aligned16(positions) || !aligned16(rope_table)) return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (n_pos < 1 || n_pos > kMaxDim) return fail(FN_E_SHAPE, "n_pos must be in [1, 2^31-1] (got %lld)", (long long)n_pos);
  if (rot_dim < 4 || rot_dim % 4 || rot_dim > head_dim)
    return fail(FN_E_SHAPE, "rot_dim must be a multiple of 4 in [4, head_dim] (got %d)", rot_dim);
  if (n_pos * (int64_t)rot_dim > (int64_t(1) << 40)) return fail(FN_E_SHAPE, "rope table above 2^40 elements");
  fn::GemmArgs rope{};
  rope.pos = positions;
  rope.rope = rope_table;
  rope.n_pos = n_pos;
  rope.rot_dim = rot_dim;
  return qknorm_impl(x, x_dtype, M, K, W_qkv, w_dtype, n_q_heads, n_kv_heads, head_dim, g_q, g_k, g_head_stride,
                     eps_x, eps_head, v_mode, &rope, g1, y, y_dtype, variant, ws, ws_bytes, stream);
}

int fn_rope_table(double base, int rot_dim, int64_t n_pos, float* table, void* stream) {
  if (!table) return fail(FN_E_NULL, "table is NULL");
  if (!aligned16(table)) return fail(FN_E_ALIGN, "table must be 16-byte aligned");
  if (!(base > 1.0) || !std::isfinite(base)) return fail(FN_E_ARG, "base must be finite and > 1");
  if (rot_dim < 2 || rot_dim % 2) return fail(FN_E_SHAPE, "rot_dim must be even and >= 2 (got %d)", rot_dim);
  if (n_pos < 0 || n_pos > kMaxDim) return fail(FN_E_SHAPE, "n_pos must be in [0, 2^31-1]");
  if (n_pos * (int64_t)rot_dim > (int64_t(1) << 40)) return fail(FN_E_SHAPE, "rope table above 2^40 elements");
  if (n_pos == 0) return ok();
  hipError_t e = fn::launch_rope_table(base, rot_dim, n_pos, table, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope table kernel launch");
  return ok();
}

int fn_fold_layernorm(const void* W, int w_dtype, const float* g, const float* beta, const float* bias, int64_t N,
                      int64_t K, void* W_star, int out_dtype, float* colsum, float* b_star, void* stream) {
  if (N < 0 || K < 0) return fail(FN_E_SHAPE, "N and K must be >= 0");
  if (N > kMaxDim || K > kMaxDim || N * K > (int64_t(1) << 40)) return fail(FN_E_SHAPE, "weight too large");
  if ((w_dtype != FN_F32 && w_dtype != FN_BF16) || (out_dtype != FN_F32 && out_dtype != FN_BF16))
    return fail(FN_E_DTYPE, "dtypes must be FN_F32 or FN_BF16");
  if (N == 0) return ok();
  if (!W || !g || !W_star || !colsum || !b_star) return fail(FN_E_NULL, "W, g, W_star, colsum and b_star are required");
  if (!aligned16(W) || !aligned16(g) || !aligned16(W_star) || (beta && !aligned16(beta)))
    return fail(FN_E_ALIGN, "W, g, beta and W_star must be 16-byte aligned");
  const int vec = (w_dtype == FN_BF16 || out_dtype == FN_BF16) ? 8 : 4;
  if (K % vec) return fail(FN_E_ALIGN, "K=%lld must be a multiple of %d", (long long)K, vec);
  const size_t in_b = (size_t)N * K * (w_dtype == FN_BF16 ? 2 : 4);
  const size_t out_b = (size_t)N * K * (out_dtype == FN_BF16 ? 2 : 4);
  const uintptr_t a0 = (uintptr_t)W, a1 = a0 + in_b, b0 = (uintptr_t)W_star, b1 = b0 + out_b;
  const bool overlap = a0 < b1 && b0 < a1;
  if (overlap && !(a0 == b0 && w_dtype == out_dtype))
    return fail(FN_E_ARG, "W_star may alias W only exactly and with equal dtypes");
  auto hits = [&](const void* v, size_t bytes) {
    const uintptr_t c0 = (uintptr_t)v, c1 = c0 + bytes;
    return (c0 < a1 && a0 < c1) || (c0 < b1 && b0 < c1);
  };
  const size_t vb = (size_t)N * 4;
  if (hits(colsum, vb) || hits(b_star, vb) ||
      ((uintptr_t)colsum < (uintptr_t)b_star + vb && (uintptr_t)b_star < (uintptr_t)colsum + vb))
    return fail(FN_E_ARG, "colsum and b_star must not overlap each other or the weights");
  hipError_t e = fn::launch_fold_layernorm(W, w_dtype, g, beta, bias, N, K, W_star, out_dtype, colsum, b_star,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fold_layernorm kernel launch");
  return ok();
}

int fn_layernorm_linear(const void* x, int x_dtype, int64_t M, int64_t K, const void* W, int w_dtype, int64_t N,
                        const float* colsum, const float* b_star, const float* g, const float* beta,
                        const float* bias, float eps, void* y, int y_dtype, int variant, void* ws, size_t ws_bytes,
                        void* stream) {
  if (int s = check_dims(M, K, N)) return s;
  if (int s = check_dtype_triple(x_dtype, w_dtype, y_dtype)) return s;
  const bool packed = variant == FN_FUSED_PACKED;
  if (packed) {
    if (int s = check_packed(M, x_dtype)) return s;
    variant = FN_FUSED;
  }
  if (variant != FN_FUSED && variant != FN_UNFUSED) {
    if (variant == FN_TWO_STREAM) return fail(FN_E_UNSUPPORTED, "the two-stream variant is offered for fn_norm_linear only");
    return fail(FN_E_ARG, "variant %d", variant);
  }
  if (!W || (M > 0 && (!x || !y))) return fail(FN_E_NULL, "W is required, and x and y when M > 0");
  for (const void* q : {(const void*)colsum, (const void*)b_star, (const void*)g, (const void*)beta, (const void*)bias})
    if (q && !aligned16(q)) return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (!aligned16(x) || !aligned16(W) || !aligned16(y)) return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (int s = check_k_vec(x_dtype, K)) return s;
  if (int s = check_eps(eps, "eps")) return s;
  if (variant == FN_FUSED) {
    if (!colsum) return fail(FN_E_NULL, "the fused variant needs colsum (from fn_fold_layernorm)");
    if (g || beta || bias) return fail(FN_E_ARG, "the fused variant takes folded parameters; g, beta and bias must be NULL");
  } else {
    if (!g) return fail(FN_E_NULL, "the unfused variant needs the gain g");
    if (colsum || b_star) return fail(FN_E_ARG, "the unfused variant takes the unfolded parameters; colsum and b_star must be NULL");
  }
  if (int s = check_ws(FN_OP_LAYERNORM_LINEAR, variant, M, K, N, x_dtype, ws, ws_bytes)) return s;
  if (M == 0) return ok();
  if (log_on())
    fprintf(stderr, "[flashnorm] layernorm_linear M=%lld K=%lld N=%lld -> %s\n", (long long)M, (long long)K,
            (long long)N, describe(fn::EPI_LN, variant, M, K, N, x_dtype, y_dtype).c_str());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fused = variant == FN_FUSED;
  const void* xin = x;
  hipError_t e;
  if (!fused) {
    e = fn::launch_layernorm(x, x_dtype == FN_BF16 ? 1 : 0, g, beta, M, K, eps, ws, st);
    if (e != hipSuccess) return hip_fail(e, "layernorm kernel launch");
    xin = ws;
  }
  const float* out_bias = fused ? b_star : bias;
  if (x_dtype == FN_F32) {
    fn::GemmF32Args a{static_cast<const float*>(xin), static_cast<const float*>(W), static_cast<float*>(y), (int)M,
                      (int)K, (int)N, eps, 1.0f / (float)K, fused ? colsum : nullptr, out_bias};
    e = fn::launch_gemm_f32(fn::EPI_LN, fused, a, st);
    if (e != hipSuccess) return hip_fail(e, "gemm_f32 kernel launch");
    return ok();
  }
  fn::GemmArgs ln{};
  ln.ln_c = fused ? colsum : nullptr;
  ln.ln_b = out_bias;
  if (fused && use_prestats(FN_OP_LAYERNORM_LINEAR, M, K, N, x_dtype)) {
    float* mu = static_cast<float*>(ws);
    float* sc = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up((size_t)M * 4));
    e = fn::launch_ln_stats(x, 1, M, K, eps, mu, sc, st);
    if (e != hipSuccess) return hip_fail(e, "ln_stats kernel launch");
    ln.row_s = sc;
    ln.row_mu = mu;
    return run_bf16(fn::EPI_LN, false, xin, W, nullptr, M, K, N, eps, y, y_dtype, &ln, st);
  }
  return run_bf16(fn::EPI_LN, fused, xin, W, nullptr, M, K, N, eps, y, y_dtype, &ln, st, packed);
}

int fn_quantize_fp8(const void* W_star, int w_dtype, int64_t N, int64_t K, uint8_t* codes, float* scales,
                    void* stream) {
  if (N < 0 || K < 0) return fail(FN_E_SHAPE, "N and K must be >= 0");
  if (N > kMaxDim || K > kMaxDim || N * K > (int64_t(1) << 40)) return fail(FN_E_SHAPE, "weight too large");
  if (w_dtype != FN_F32 && w_dtype != FN_BF16) return fail(FN_E_DTYPE, "w_dtype must be FN_F32 or FN_BF16");
  if (N == 0) return ok();
  if (!W_star || !codes || !scales) return fail(FN_E_NULL, "W_star, codes and scales are required");
  if (!aligned16(W_star) || !aligned16(codes) || !aligned16(scales)) return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (K == 0 || K % 16) return fail(FN_E_ALIGN, "K=%lld must be a positive multiple of 16", (long long)K);
  const uintptr_t a0 = (uintptr_t)W_star, a1 = a0 + (size_t)N * K * (w_dtype == FN_BF16 ? 2 : 4);
  const uintptr_t c0 = (uintptr_t)codes, c1 = c0 + (size_t)N * K, s0 = (uintptr_t)scales, s1 = s0 + (size_t)N * 4;
  if ((c0 < a1 && a0 < c1) || (s0 < a1 && a0 < s1) || (s0 < c1 && c0 < s1))
    return fail(FN_E_ARG, "codes, scales and W_star must not overlap");
  hipError_t e = fn::launch_quantize_fp8(W_star, w_dtype, N, K, codes, scales, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize_fp8 kernel launch");
  return ok();
}

int fn_decode_packed_bytes(int w_dtype, int64_t N, int64_t K, size_t* out_bytes) {
  if (!out_bytes) return fail(FN_E_NULL, "out_bytes is NULL");
  if (w_dtype != FN_BF16 && w_dtype != FN_E4M3) return fail(FN_E_DTYPE, "w_dtype must be FN_BF16 or FN_E4M3");
  if (N < 0 || K < 1) return fail(FN_E_SHAPE, "need N >= 0 and K >= 1");
  if (N > kMaxDim || K > kMaxDim || N * K > (int64_t(1) << 40)) return fail(FN_E_SHAPE, "weight too large");
  if (K % (w_dtype == FN_BF16 ? 8 : 16))
    return fail(FN_E_ALIGN, "K=%lld must be a multiple of %d", (long long)K, w_dtype == FN_BF16 ? 8 : 16);
  const int64_t row_bytes = K * (w_dtype == FN_BF16 ? 2 : 1);
  *out_bytes = (size_t)((N + 15) / 16) * (size_t)((row_bytes + 63) / 64) * 1024;
  return ok();
}

int fn_pack_decode_weights(const void* W, int w_dtype, int64_t N, int64_t K, void* W_packed, void* stream) {
  size_t bytes = 0;
  if (int s = fn_decode_packed_bytes(w_dtype, N, K, &bytes)) return s;
  if (N == 0) return ok();
  if (!W || !W_packed) return fail(FN_E_NULL, "W and W_packed are required");
  if (!aligned16(W) || !aligned16(W_packed)) return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  const int64_t row_bytes = K * (w_dtype == FN_BF16 ? 2 : 1);
  const uintptr_t a0 = (uintptr_t)W, a1 = a0 + (size_t)N * row_bytes;
  const uintptr_t p0 = (uintptr_t)W_packed, p1 = p0 + bytes;
  if (p0 < a1 && a0 < p1) return fail(FN_E_ARG, "W and W_packed must not overlap");
  hipError_t e = fn::launch_pack_decode(W, nullptr, N, row_bytes, W_packed, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack_decode kernel launch");
  return ok();
}

int fn_pack_decode_weights_glu(const void* W_gate, const void* W_up, int w_dtype, int64_t N, int64_t K,
                               void* W_packed, void* stream) {
  size_t bytes = 0;
  if (int s = fn_decode_packed_bytes(w_dtype, N, K, &bytes)) return s;
  if (N == 0) return ok();
  if (!W_gate || !W_up || !W_packed) return fail(FN_E_NULL, "W_gate, W_up and W_packed are required");
  if (!aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_packed))
    return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  const int64_t row_bytes = K * (w_dtype == FN_BF16 ? 2 : 1);
  const uintptr_t p0 = (uintptr_t)W_packed, p1 = p0 + 2 * bytes;
  for (const void* w : {W_gate, W_up}) {
    const uintptr_t a0 = (uintptr_t)w, a1 = a0 + (size_t)N * row_bytes;
    if (p0 < a1 && a0 < p1) return fail(FN_E_ARG, "W_packed must not overlap W_gate or W_up");
  }
  hipError_t e = fn::launch_pack_decode(W_gate, W_up, N, row_bytes, W_packed, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack_decode kernel launch");
  return ok();
}

int fn_norm_linear_fp8(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* W8, const float* w_scales,
                       int64_t N, const float* g, float eps, void* y, int y_dtype, int variant, void* ws,
                       size_t ws_bytes, void* stream) {
  return fp8_impl(FN_OP_NORM_LINEAR_FP8, x, x_dtype, M, K, W8, w_scales, nullptr, nullptr, N, g, eps, y, y_dtype,
                  variant, ws, ws_bytes, stream);
}

int fn_norm_glu_ffn_fp8(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* W8_gate,
                        const float* s_gate, const uint8_t* W8_up, const float* s_up, int64_t N, const float* g,
                        float eps, void* h, int h_dtype, int variant, void* ws, size_t ws_bytes, void* stream) {
  if (!s_up || (!W8_up && variant != FN_FUSED_PACKED))
    return fail(FN_E_NULL, "W8_up and s_up are required (W8_up NULL only with a packed gate/up pair)");
  return fp8_impl(FN_OP_NORM_GLU_FFN_FP8, x, x_dtype, M, K, W8_gate, s_gate, W8_up, s_up, N, g, eps, h, h_dtype,
                  variant, ws, ws_bytes, stream);
}

int fn_linear_latent_norm(const void* x, int x_dtype, int64_t M, int64_t K, const void* W, int w_dtype,
                          int64_t n_q_latent, int64_t n_kv_latent, int64_t n_rope, const float* g_q_latent,
                          const float* g_kv_latent, float eps_x, float eps_latent, const int32_t* positions,
                          const float* rope_table, int64_t n_pos, int rot_dim, const float* g1, void* y, int y_dtype,
                          int variant, void* ws, size_t ws_bytes, void* stream) {
  if (n_q_latent < 0 || n_kv_latent < 0 || n_rope < 0) return fail(FN_E_SHAPE, "segment widths must be >= 0");
  if (n_q_latent % 32 || n_kv_latent % 32) return fail(FN_E_SHAPE, "latent widths must be multiples of 32");
  if (n_rope % 4) return fail(FN_E_SHAPE, "n_rope must be a multiple of 4");
  if (n_q_latent + n_kv_latent == 0) return fail(FN_E_SHAPE, "at least one latent is required");
  const int64_t N = n_q_latent + n_kv_latent + n_rope;
  if (int s = check_dims(M, K, N)) return s;
  if (int s = check_dtype_triple(x_dtype, w_dtype, y_dtype)) return s;
  if (x_dtype != FN_BF16) return fail(FN_E_UNSUPPORTED, "the latent-norm op is bf16 only");
  if (variant != FN_FUSED && variant != FN_UNFUSED) {
    if (variant == FN_FUSED_PACKED) return fail(FN_E_UNSUPPORTED, "decode-packed weights: plain, glu or LayerNorm ops only");
    if (variant == FN_TWO_STREAM) return fail(FN_E_UNSUPPORTED, "the two-stream variant is offered for fn_norm_linear only");
    return fail(FN_E_ARG, "variant %d", variant);
  }
  if (!W || (M > 0 && (!x || !y))) return fail(FN_E_NULL, "W is required, and x and y when M > 0");
  if ((n_q_latent && !g_q_latent) || (n_kv_latent && !g_kv_latent)) return fail(FN_E_NULL, "each latent needs its gain");
  for (const void* q : {(const void*)x, (const void*)W, (const void*)y, (const void*)g_q_latent,
                        (const void*)g_kv_latent, (const void*)positions, (const void*)rope_table, (const void*)g1})
    if (q && !aligned16(q)) return fail(FN_E_ALIGN, "pointers must be 16-byte aligned");
  if (int s = check_k_vec(x_dtype, K)) return s;
  if (int s = check_eps(eps_x, "eps_x")) return s;
  if (int s = check_eps(eps_latent, "eps_latent")) return s;
  if (positions) {
    if (!rope_table) return fail(FN_E_NULL, "rope_table is required with positions");
    if (n_pos < 1 || n_pos > kMaxDim) return fail(FN_E_SHAPE, "n_pos must be in [1, 2^31-1]");
    if (rot_dim < 4 || rot_dim % 4 || rot_dim > n_rope)
      return fail(FN_E_SHAPE, "rot_dim must be a multiple of 4 in [4, n_rope] (got %d)", rot_dim);
  }
  if (variant == FN_UNFUSED && !g1) return fail(FN_E_NULL, "the unfused variant needs the first norm's gain g1");
  if (variant == FN_FUSED && g1) return fail(FN_E_ARG, "the fused variant takes the folded W; g1 must be NULL");
  if (int s = check_ws(FN_OP_LINEAR_LATENT_NORM, variant, M, K, N, x_dtype, ws, ws_bytes)) return s;
  if (M == 0) return ok();
  if (log_on())
    fprintf(stderr, "[flashnorm] linear_latent_norm M=%lld K=%lld N=%lld -> %s\n", (long long)M, (long long)K,
            (long long)N, describe(fn::EPI_LATENT, variant, M, K, N, x_dtype, y_dtype).c_str());
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* wsc = static_cast<char*>(ws);
  const void* xin = x;
  if (variant == FN_UNFUSED) {
    hipError_t e = fn::launch_rmsnorm(x, 1, g1, M, K, eps_x, wsc, st);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm kernel launch");
    xin = wsc;
    wsc += round_up((size_t)M * K * 2);
  }
  const int lat = (int)(n_q_latent + n_kv_latent);
  fn::GemmArgs a{};
  a.lat_cols = lat;
  a.lat_z = reinterpret_cast<float*>(wsc);
  a.lat_part = reinterpret_cast<float*>(wsc + round_up((size_t)M * N * 4));
  bool sums_inside = variant == FN_FUSED;
  if (variant == FN_FUSED && use_prestats(FN_OP_LINEAR_LATENT_NORM, M, K, N, x_dtype)) {
    float* srow = reinterpret_cast<float*>(wsc + latent_ws(M, N));
    hipError_t e = fn::launch_row_scale(x, 1, M, K, eps_x, srow, st);
    if (e != hipSuccess) return hip_fail(e, "row_scale kernel launch");
    a.row_s = srow;
    sums_inside = false;
  }
  a.pos = positions;
  a.rope = rope_table;
  a.n_pos = n_pos;
  a.rot_dim = rot_dim;
  if (int s = run_bf16(fn::EPI_LATENT, sums_inside, xin, W, nullptr, M, K, N, eps_x, y, y_dtype, &a, st))
    return s;
  hipError_t e = fn::launch_latent_norm(a.lat_z, a.lat_part, M, lat, (int)n_q_latent, g_q_latent, g_kv_latent,
                                        eps_latent, y, N, y_dtype, st);
  if (e != hipSuccess) return hip_fail(e, "latent_norm kernel launch");
  return ok();
}

int fn_norm_linear_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, const void* W_star, int w_dtype,
                           int64_t N, float eps, void* y, int y_dtype, void* stream) {
  // Everything fn_norm_linear checks, on the fused variant, before the
  // scratch is touched; then the scratch's size.
  if (int s = check_dims(M, K, N)) return s;
  if (int s = check_dtype_triple(x_dtype, w_dtype, y_dtype)) return s;
  size_t need = 0;
  if (x_dtype == FN_BF16 || x_dtype == FN_F32) need = ws_need(FN_OP_NORM_LINEAR, FN_FUSED, M, K, N, x_dtype);
  if (need > kScratchBytes)
    return fail(FN_E_WORKSPACE, "this shape needs %zu bytes of scratch; the library's static scratch holds %zu "
                "(use fn_norm_linear with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0 && M > 0 && x && W_star && y) {
    hipError_t e;
    ws = scratch_on_current_device(&e);
    if (!ws) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  }
  return fn_norm_linear(x, x_dtype, M, K, W_star, w_dtype, N, nullptr, eps, y, y_dtype, FN_FUSED, ws,
                        ws ? kScratchBytes : 0, stream, nullptr);
}

void fn_shutdown(void) { g_events.release(); }

int fn_testing_skip_join(int skip) {
  const int was = g_skip_join ? 1 : 0;
  g_skip_join = skip != 0;
  return was;
}

int fn_testing_gemm_events(void* const* starts, void* const* stops, int n) {
  g_gemm_timing = GemmTiming{};
  if (n <= 0) return ok();
  if (starts == nullptr || stops == nullptr) return fail(FN_E_NULL, "fn_testing_gemm_events: NULL event arrays");
  g_gemm_timing.starts = starts;
  g_gemm_timing.stops = stops;
  g_gemm_timing.n = n;
  return ok();
}

}  // extern "C"
