/*
 * flashnorm.h -- C ABI of the MI355X (gfx950) FlashNorm norm-then-project
 * library, libflashnorm.so.
 *
 * The method (FlashNorm: Fast Normalization for Transformers, Abstract):
 * an RMSNorm followed by a linear layer is rewritten exactly as
 *   (i)  the RMSNorm gain g folded offline into the weight, W* = W diag(g)
 *        in checkpoint layout, and
 *   (ii) the per-row 1/RMS scalar applied to the *output* of the matrix
 *        product, so the row sum of squares runs alongside the contraction:
 *          y[m,n] = s[m] * sum_k x[m,k] W*[n,k],
 *          s[m]   = 1 / sqrt(mean_k x[m,k]^2 + eps).
 * An RMSNorm -> linear -> RMSNorm chain may drop its first RMSNorm by scale
 * invariance (same Abstract); fn_linear_qknorm does that for q/k heads and
 * fn_linear_latent_norm for the latents of MLA attention.  The same
 * rewrite covers LayerNorm (fn_layernorm_linear), RoPE after the head norms
 * (fn_linear_qknorm_rope) and fp8 folded weights with fp8 or bf16
 * activations (fn_norm_linear_fp8).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout    All tensors are dense row-major.  x is [M x K]; weights are
 *            [N x K] (out features x in features, K contiguous: the layout
 *            a linear layer's weight has in a checkpoint, so the layer is
 *            x . W^T); outputs are [M x N_out]; gains are float32 vectors.
 *  Pointers  Device pointers (HBM) unless stated.  The caller owns every
 *            buffer; the library never allocates or frees device memory.
 *  Alignment Every device pointer must be 16-byte aligned and K a multiple
 *            of 8 (bf16) or 4 (f32), 16 for fp8 weights, else FN_E_ALIGN.
 *            bf16 calls take K <= 2^21 (FN_E_UNSUPPORTED above).
 *  Streams   `stream` is a hipStream_t passed as void* (NULL = the null
 *            stream).  All work is enqueued on it, in order; no call blocks
 *            the host.  The two-stream variant also uses `stream_aux`, and
 *            forks from / joins back to `stream` with events, so to the
 *            caller it is ordered exactly like a single-stream call.
 *  Errors    Every argument is validated before anything is launched; a
 *            call that returns an error has launched nothing and written
 *            nothing.  A failed launch returns FN_E_HIP.  fn_last_error()
 *            gives a message for the calling thread's last error.  Faults
 *            inside a kernel surface at the caller's next synchronisation.
 *  Threads   Entry points are re-entrant; concurrent calls on one stream
 *            are ordered by that stream.
 *  Dtypes    (x, W, y) triples: (F32, F32, F32) and (BF16, BF16, BF16|F32);
 *            the fp8 entry points take bf16 x, E4M3 weight codes (bytes)
 *            with float32 channel scales, and F32 or BF16 y.  Products
 *            accumulate in float32.
 *  M = 0     is allowed and launches nothing; the per-row pointers (x, y,
 *            h, positions) may then be NULL, as an empty tensor's are.
 *  Tuning    The prefill tile is chosen from M and N (see fn_dispatch_name).
 *            The environment variable FN_TILE=<n> forces tile n of the
 *            build's table for every bf16 prefill call (a tuning aid; an
 *            unknown n, or a tile the op cannot use, is ignored).
 *            FN_PRESTATS=0 / 1 turns the fused variant's row-statistics
 *            pass off / on for every bf16 fn_norm_linear,
 *            fn_layernorm_linear and fn_linear_latent_norm call with
 *            M > 16 (the workspace size follows; query it under the same
 *            setting).  FN_DECODE_ORDER=consec / rr forces the order in
 *            which the bf16 weight-streaming kernel (M <= 16) deals K steps
 *            to its waves: consecutive steps, or round-robin.  The result
 *            may differ in the last bits between the two orders.
 */
#ifndef FLASHNORM_H
#define FLASHNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FN_ABI_VERSION 3

typedef enum {
  FN_OK = 0,
  FN_E_NULL = 1,        /* a required pointer is NULL                  */
  FN_E_SHAPE = 2,       /* a size is negative, zero where not allowed, or inconsistent */
  FN_E_DTYPE = 3,       /* unsupported dtype or dtype combination      */
  FN_E_ALIGN = 4,       /* pointer not 16-byte aligned or K not a multiple of the vector width */
  FN_E_WORKSPACE = 5,   /* workspace missing or smaller than fn_workspace_bytes() */
  FN_E_UNSUPPORTED = 6, /* valid request that the library does not implement */
  FN_E_HIP = 7,         /* a HIP runtime call or launch failed         */
  FN_E_ARG = 8          /* any other invalid argument (variant, v_mode, eps < 0, ...) */
} fn_status;

typedef enum {
  FN_F32 = 0,
  FN_BF16 = 1,
  FN_E4M3 = 2 /* fp8 weight codes (bytes); a w_dtype of fn_decode_packed_bytes / fn_pack_decode_weights */
} fn_dtype;

typedef enum {
  FN_FUSED = 0,      /* folded weight, deferred row scale (one kernel; large shapes: a
                        row-statistics pass, then the GEMM with the scale in its epilogue) */
  FN_UNFUSED = 1,    /* baseline: RMSNorm kernel writes xn, then the GEMM on the unfolded W */
  FN_TWO_STREAM = 2, /* GEMM on stream_aux, sum of squares on stream, explicit event join, post-scale */
  FN_FUSED_PACKED = 3 /* FN_FUSED with the weights in the decode-packed layout (fn_pack_decode_weights):
                         bf16 x, M <= 16, fn_norm_linear / fn_norm_glu_ffn / fn_layernorm_linear and
                         the fp8 ops; other ops and larger M return FN_E_UNSUPPORTED */
} fn_variant;

typedef enum {
  FN_OP_NORM_LINEAR = 0,
  FN_OP_NORM_GLU_FFN = 1,
  FN_OP_LINEAR_QKNORM = 2,
  FN_OP_LINEAR_QKNORM_ROPE = 3,
  FN_OP_LAYERNORM_LINEAR = 4,
  FN_OP_NORM_LINEAR_FP8 = 5,
  FN_OP_NORM_GLU_FFN_FP8 = 6,
  FN_OP_LINEAR_LATENT_NORM = 7
} fn_op;

/* Version of this ABI (FN_ABI_VERSION of the build). */
int fn_abi_version(void);

/* Message for the calling thread's most recent non-FN_OK status ("" if none).
 * The string stays valid until the next call on the same thread. */
const char* fn_last_error(void);

/* Static name of a status code. */
const char* fn_status_string(int status);

/* Bytes of device workspace `op` needs for `variant` at this shape
 * (N = output columns of one projection; for the qknorm ops the total
 * q+k+v width).  Writes *out_bytes.  FN_FUSED needs 0 except where it
 * takes the row-statistics pass (bf16 fn_norm_linear / fn_layernorm_linear
 * with at least 240 tiles of 256 x 256 outputs): then M floats of row
 * scales (and, for LayerNorm, M row means), each 256-byte padded; and for
 * the head-norm ops at M <= 16, where the weight-streaming kernel writes the
 * float32 product (M x N floats, 256-byte padded) before the per-head pass
 * (after the normalised activations for FN_UNFUSED). */
int fn_workspace_bytes(int op, int variant, int64_t M, int64_t K, int64_t N, int x_dtype,
                       size_t* out_bytes);

/* Name of the kernel configuration a call with these arguments dispatches
 * to (for logs and tests).  Writes a NUL-terminated string of at most
 * `len` bytes into `buf` (host memory). */
int fn_dispatch_name(int op, int variant, int64_t M, int64_t K, int64_t N, int x_dtype, int y_dtype,
                     char* buf, size_t len);

/*
 * Offline weight fold (FlashNorm Abstract, point (i); the summary page's
 * "Weight Folding" bullet: the normalisation gain is folded into the
 * projection weights offline).
 *   W_star[n,k] = round(g[k] * W[n,k])
 * The product is formed exactly (in float64) and rounded once, to nearest
 * with ties to even, to out_dtype.
 *   W      [N x K], w_dtype in {F32, BF16}, device
 *   g      [K] float32, device
 *   W_star [N x K], out_dtype in {F32, BF16}, device; may alias W when the
 *          dtypes are equal (in-place fold), must not partially overlap it.
 */
int fn_fold_weights(const void* W, int w_dtype, const float* g, int64_t N, int64_t K,
                    void* W_star, int out_dtype, void* stream);

/*
 * RMSNorm followed by a bias-free linear layer (FlashNorm Abstract, points
 * (i) and (ii)).
 *   x [M x K] (x_dtype), W [N x K] (w_dtype == x_dtype), y [M x N] (y_dtype)
 *   FN_FUSED, FN_TWO_STREAM: W is the folded W*; g must be NULL.
 *       y = (x . W*^T) * s[m],  s[m] = 1/sqrt(mean_k x[m,k]^2 + eps)
 *       FN_FUSED takes the row sums of squares alongside the contraction,
 *       or (large bf16 shapes, see fn_workspace_bytes) in one pass over x
 *       before it, writing s into the workspace; either way x is never
 *       normalised in memory and s multiplies the product's output.
 *   FN_UNFUSED: W is the unfolded weight and g [K] float32 is required.
 *       xn = RMSNorm(x; g) rounded to x_dtype (workspace), then y = xn . W^T
 *   FN_FUSED_PACKED: as FN_FUSED with W* in the decode-packed layout
 *       (fn_pack_decode_weights); bf16, M <= 16.  The same holds for
 *       fn_norm_glu_ffn (both weights packed, or the pair layout of
 *       fn_pack_decode_weights_glu as W_gate with W_up NULL),
 *       fn_layernorm_linear and the fp8 ops (packed codes, row-major scales).
 *   eps >= 0 (eps == 0 with an all-zero row gives NaN, as the definition does).
 *   ws / ws_bytes: device workspace of at least fn_workspace_bytes() bytes
 *       (may be NULL when that is 0).
 *   stream_aux: FN_TWO_STREAM only (must differ from stream); ignored otherwise.
 *       The aux stream runs the GEMM into a float32 workspace, the main
 *       stream the row sum of squares; the post-scale waits on events
 *       recorded at the end of both (the explicit join whose absence lets a
 *       post-scale read a stale product, the race the talk pages describe).
 */
int fn_norm_linear(const void* x, int x_dtype, int64_t M, int64_t K,
                   const void* W, int w_dtype, int64_t N,
                   const float* g, float eps,
                   void* y, int y_dtype, int variant,
                   void* ws, size_t ws_bytes, void* stream, void* stream_aux);

/*
 * RMSNorm followed by the gate and up projections of a SiLU-gated FFN
 * (FlashNorm Abstract: the techniques extend to FFNs with GLU variants).
 *   h[m,n] = SiLU(s[m] * a[m,n]) * (s[m] * b[m,n]),
 *   a = x . W_gate*^T, b = x . W_up*^T  (FN_FUSED; both weights folded)
 *   FN_UNFUSED: unfolded W_gate / W_up and g [K] float32; xn as above.
 *   W_gate, W_up [N x K]; h [M x N].  FN_TWO_STREAM is not offered here.
 * Rows M <= 16 dispatch to a weight-streaming decode kernel.
 */
int fn_norm_glu_ffn(const void* x, int x_dtype, int64_t M, int64_t K,
                    const void* W_gate, const void* W_up, int w_dtype, int64_t N,
                    const float* g, float eps, void* h, int h_dtype, int variant,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * Attention input projection with per-head RMSNorm on q and k, the
 * pre-attention RMSNorm dropped by scale invariance (FlashNorm Abstract:
 * RMSNorm -> linear -> RMSNorm lets the first RMSNorm be eliminated, which
 * removes the pre-attention RMSNorm of QKV-normalised models).
 *   W_qkv [N x K], N = (n_q_heads + 2 n_kv_heads) * head_dim, output columns
 *   ordered [q heads | k heads | v heads]; head_dim in {64, 128, 256}.
 *   FN_FUSED: W_qkv is folded with the first RMSNorm's gain; g1 must be NULL.
 *     z = x . W_qkv*^T
 *     q/k head h: y = z_h * g_{q|k} / sqrt(mean(z_h^2) + eps_head)
 *     v heads:    v_mode 0: y = z_v * s[m], s[m] = 1/sqrt(mean_k x^2 + eps_x)
 *                 v_mode 1: y = z_v / sqrt(mean(z_v^2) + eps_head) (unit gain)
 *   FN_UNFUSED: unfolded W_qkv and g1 [K]; xn = RMSNorm(x; g1, eps_x) is
 *     materialised, then the same head norms on xn . W_qkv^T (v: no scale).
 *   g_q, g_k: float32 gains, [head_dim] shared by all heads when
 *     g_head_stride == 0, else head h uses g + h * g_head_stride.
 *   M <= 16: the weight-streaming kernel writes z (float32) to the
 *     workspace (see fn_workspace_bytes) and a per-(row, head) pass applies
 *     the head norms; the same arithmetic as the head-norm tile's epilogue.
 *   FN_TWO_STREAM is not offered here.
 */
int fn_linear_qknorm(const void* x, int x_dtype, int64_t M, int64_t K,
                     const void* W_qkv, int w_dtype, int n_q_heads, int n_kv_heads, int head_dim,
                     const float* g_q, const float* g_k, int64_t g_head_stride,
                     float eps_x, float eps_head, int v_mode,
                     const float* g1, void* y, int y_dtype, int variant,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * fn_linear_qknorm followed by the rotary position embedding of every q and
 * k head (FlashNorm Abstract: the techniques extend to RoPE-based attention;
 * the rotation is the one defined in RoFormer: Enhanced Transformer with
 * Rotary Position Embedding, Section 3.2).  The per-head norm, its gain and
 * then the rotation all happen in the projection's epilogue:
 *   q/k head h of row m: y_h = R(positions[m]) (z_h * g / sqrt(mean(z_h^2) + eps_head))
 * where R turns column pair (2i, 2i+1), i < rot_dim/2, of the head by the
 * angle positions[m] * theta_i:  (a, b) -> (a cos - b sin, a sin + b cos),
 * and leaves columns rot_dim .. head_dim-1 as they are.  v heads are not
 * rotated.  Every other argument is as for fn_linear_qknorm.
 *   positions  [M] int32, device: the token position of each row.  A
 *              position outside [0, n_pos) gives NaN in that row's q and k
 *              (nothing outside the table is read).
 *   rope_table [n_pos x rot_dim] float32, device, 16-byte aligned: entry
 *              (p, 2i) = cos(p theta_i), (p, 2i+1) = sin(p theta_i), as
 *              written by fn_rope_table.
 *   rot_dim    rotated columns per head: a multiple of 4, 4 <= rot_dim <= head_dim.
 * Models whose rotation pairs column i with column i + rot_dim/2 instead
 * ("rotate half") use this entry point after permuting the q and k rows of
 * W_qkv (and the gains) so that those partners become neighbours; q.k^T, and
 * so attention, is unchanged by a permutation applied to both q and k.
 */
int fn_linear_qknorm_rope(const void* x, int x_dtype, int64_t M, int64_t K,
                          const void* W_qkv, int w_dtype, int n_q_heads, int n_kv_heads, int head_dim,
                          const float* g_q, const float* g_k, int64_t g_head_stride,
                          float eps_x, float eps_head, int v_mode,
                          const int32_t* positions, const float* rope_table, int64_t n_pos, int rot_dim,
                          const float* g1, void* y, int y_dtype, int variant,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Rotary table for fn_linear_qknorm_rope (set-up, like the weight fold):
 *   table[p * rot_dim + 2i]     = cos(p * theta_i)
 *   table[p * rot_dim + 2i + 1] = sin(p * theta_i),   theta_i = base^(-2i / rot_dim),
 * for 0 <= p < n_pos and 0 <= i < rot_dim/2 (RoFormer, Section 3.2).  Angle,
 * cosine and sine are computed in float64 and rounded once to float32.
 *   base > 1 (10000 in RoFormer), rot_dim even, table device memory of
 *   n_pos * rot_dim floats, 16-byte aligned.  n_pos == 0 writes nothing.
 */
int fn_rope_table(double base, int rot_dim, int64_t n_pos, float* table, void* stream);

/*
 * Offline fold for fn_layernorm_linear (FlashNorm Abstract: the same
 * techniques extend to LayerNorm; LayerNorm as in Layer Normalization, Ba,
 * Kiros and Hinton, Section 3):
 *   W_star[n,k] = round(g[k] * W[n,k])      exactly as fn_fold_weights
 *   colsum[n]   = sum_k W_star[n,k]         over the stored (rounded) W_star
 *   b_star[n]   = sum_k beta[k] W[n,k] + bias[n]
 * Both sums run in float64 and are rounded once to float32.
 *   W [N x K] (w_dtype), g [K] float32, beta [K] float32 or NULL (zero),
 *   bias [N] float32 or NULL (zero): the LayerNorm's gain and bias and the
 *   linear layer's bias.  W_star [N x K] (out_dtype) may alias W exactly
 *   when the dtypes match.  colsum, b_star: [N] float32, device; they must
 *   not overlap each other or the weights.  K a multiple of 8 (bf16 on
 *   either side) or 4.  N == 0 does nothing.
 */
int fn_fold_layernorm(const void* W, int w_dtype, const float* g, const float* beta, const float* bias,
                      int64_t N, int64_t K, void* W_star, int out_dtype, float* colsum, float* b_star,
                      void* stream);

/*
 * LayerNorm followed by a linear layer with bias, with the gain folded and
 * the normalisation deferred to the product's output:
 *   y[m,n] = s[m] (z[m,n] - mu[m] colsum[n]) + b_star[n],  z = x . W_star^T,
 *   mu[m] = mean_k x[m,k],  s[m] = 1 / sqrt(mean_k (x[m,k] - mu[m])^2 + eps),
 * which equals LayerNorm(x; g, beta) . W^T + bias.  mu and the variance
 * come from sums of x - x[m,0] and (x - x[m,0])^2 taken alongside the
 * contraction (the shift keeps the variance free of cancellation).
 *   FN_FUSED: W is W_star; colsum required and b_star optional (NULL =
 *     zero), both from fn_fold_layernorm; g, beta and bias must be NULL.
 *   FN_UNFUSED: W is the unfolded weight; g required, beta and bias
 *     optional; colsum and b_star must be NULL.  A LayerNorm kernel writes
 *     xn = LayerNorm(x) in x_dtype to the workspace, then y = xn . W^T + bias.
 *   Dtypes, layout, alignment (every non-NULL vector 16-byte aligned),
 *   workspace and errors as fn_norm_linear; M <= 16 (bf16) runs the
 *   weight-streaming decode kernel.  FN_TWO_STREAM is not offered here.
 */
int fn_layernorm_linear(const void* x, int x_dtype, int64_t M, int64_t K,
                        const void* W, int w_dtype, int64_t N,
                        const float* colsum, const float* b_star,
                        const float* g, const float* beta, const float* bias,
                        float eps, void* y, int y_dtype, int variant,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * fp8 weights (FlashNorm: the folded checkpoint stays compatible with
 * quantised models).  Offline, after the fold: per output channel n,
 *   scales[n]   = float32(float64(max_k |W[n,k]|) / 448)   (1 for a zero row)
 *   codes[n,k]  = E4M3(W[n,k] / scales[n])
 * the exact quotient rounded once to nearest, ties to even (the library
 * decides in float32 with an exact residual test; a float64 division gives
 * the same codes, and rows with a scale below 2^-96 use one), in the OCP
 * 8-bit floating point
 * E4M3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * largest finite 448), saturating at +-448.  The dequantised weight is
 * scales[n] * value(codes[n,k]).
 *   W_star [N x K] (F32 or BF16), device; codes [N x K] bytes and scales [N]
 *   float32, device, 16-byte aligned, not overlapping W_star or each other;
 *   K a multiple of 16.  N == 0 does nothing.
 */
int fn_quantize_fp8(const void* W_star, int w_dtype, int64_t N, int64_t K, uint8_t* codes, float* scales,
                    void* stream);

/*
 * Decode-packed weight layout, read by the weight-streaming (decode) kernel
 * for M <= 16 rows under FN_FUSED_PACKED.  A decode step streams every
 * weight byte once, so its speed is the rate at which the chip reads the
 * weights; in the row-major layout one wave load gathers 64 bytes from each
 * of 16 rows, in this layout it reads 1 KB of contiguous memory.  It is a
 * re-layout of the folded weight (or of its fp8 codes), done once offline
 * like the fold itself; the operation is unchanged (FlashNorm Abstract,
 * points (i) and (ii)).  The result is FN_FUSED's on the row-major weight,
 * bit for bit where the two deal K steps to the waves in the same order
 * (always for fp8; bf16 glu with M > 4, bf16 plain and LayerNorm with
 * M <= 4), otherwise up to the order of the float32 sums.
 *   The [N x K] weight is cut into 16-row slabs and each row into 64-byte
 *   steps (32 bf16 or 64 fp8 values).  Step st of slab j is 64 pieces of 16
 *   bytes; piece p holds row 16 j + (p mod 16), bytes 64 st + 16 floor(p / 16)
 *   to 64 st + 16 floor(p / 16) + 15 of that row.  Byte offset of the piece:
 *     ((j * S + st) * 64 + p) * 16,   S = ceil(K * e / 64) steps per slab,
 *   e = 2 (FN_BF16) or 1 (FN_E4M3).  Rows >= N and bytes past a row's end
 *   are zero.  Size: ceil(N / 16) * S * 1024 bytes (fn_decode_packed_bytes).
 *   W [N x K] row-major, device; W_packed device, must not overlap W.
 *   K a multiple of 8 (bf16) or 16 (fp8).  N == 0 does nothing.
 * The fp8 channel scales stay [N] float32 vectors.
 * Errors: FN_E_DTYPE for a w_dtype other than FN_BF16 / FN_E4M3; FN_E_SHAPE
 * for N < 0, K < 1 or a weight above 2^40 elements; FN_E_ALIGN for K or a
 * pointer off its alignment; FN_E_NULL for a missing pointer (N > 0);
 * FN_E_ARG when W_packed overlaps W.
 */
int fn_decode_packed_bytes(int w_dtype, int64_t N, int64_t K, size_t* out_bytes);

int fn_pack_decode_weights(const void* W, int w_dtype, int64_t N, int64_t K, void* W_packed, void* stream);

/*
 * The gate/up pair layout for fn_norm_glu_ffn / fn_norm_glu_ffn_fp8: both
 * weights in one buffer, each K step of slab j holding W_gate's 64 pieces
 * (as above), then W_up's, so a workgroup reads its gate and up rows as one
 * contiguous run (2-3% faster than two packed buffers at M <= 4).
 *   byte offset of piece p of step st of slab j of W_gate:
 *     (((j * S + st) * 2) * 64 + p) * 16;  of W_up: add 1024.
 *   Size: twice fn_decode_packed_bytes.  Pass the buffer as W_gate (W8_gate)
 *   with W_up (W8_up) NULL under FN_FUSED_PACKED; the fp8 channel scales
 *   stay two [N] vectors.  W_packed must not overlap W_gate or W_up.
 *   Errors as fn_pack_decode_weights.
 */
int fn_pack_decode_weights_glu(const void* W_gate, const void* W_up, int w_dtype, int64_t N, int64_t K,
                               void* W_packed, void* stream);

/*
 * fn_norm_linear, FN_FUSED, for callers that cannot allocate memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Arguments, layouts, results and errors are those of
 * fn_norm_linear with variant FN_FUSED, g NULL and no stream_aux; the
 * workspace that call may need (the row statistics of large shapes: one
 * float32 per row) lives in a static device array of the library, 4 MiB per
 * GPU (row statistics of up to 2^20 rows), taken once per device and held
 * until the process ends.  A shape that needs more returns FN_E_WORKSPACE
 * before anything is launched.  The call allocates nothing: no hipMalloc,
 * no allocating library routine.  It uses the array of the current device,
 * which must be the device of `stream`.  Every call on a GPU shares that
 * GPU's array, so calls whose work overlaps on one GPU (other streams,
 * other threads) race; calls ordered on one stream do not.  Nothing in the
 * array needs to start at zero: each call writes every value it reads.
 */
int fn_norm_linear_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, const void* W_star, int w_dtype,
                           int64_t N, float eps, void* y, int y_dtype, void* stream);

/*
 * fn_norm_linear / fn_norm_glu_ffn on fp8 weights (the folded checkpoint
 * stays usable by quantised models: the FlashNorm talk write-up's "Results"
 * bullet; the qabash.com talk page's summary).
 *   Decode regime, M <= 16 rows: the weights stream from memory as bytes
 *   (half the bf16 traffic) and are widened to bf16 in registers (exactly)
 *   for the bf16 MFMAs:
 *     y[m,n] = s[m] * scales[n] * sum_k x[m,k] value(codes[n,k])
 *     h[m,n] = SiLU(s[m] q_g[n] a[m,n]) * (s[m] q_u[n] b[m,n])
 *   Prefill, M > 16: x is quantised per row to E4M3 too (q_x[m] =
 *   float32(amax_m / 448), codes of x / q_x rounded to nearest even, as
 *   fn_quantize_fp8 does for a weight's rows), in a pass that also takes
 *   each row's sum of squares; then one fp8 MFMA product of the two code
 *   matrices, with the row factor s[m] q_x[m] and the channel scale in its
 *   epilogue:
 *     y[m,n] = s[m] q_x[m] scales[n] * sum_k value(cx[m,k]) value(codes[n,k])
 *   (per-row quantisation does not depend on a positive row scale, so
 *   quantising x equals quantising RMSNorm(x), up to the rounding of the
 *   scales).  Workspace (fn_workspace_bytes): the M x K codes at offset 0,
 *   then at offset round_up(M K, 256) the M float32 row factors.
 *   x [M x K] bf16; y / h [M x N] (F32 or BF16); K a multiple of 16.
 *   FN_FUSED: codes and scales of the folded W* (fn_fold_weights, then
 *     fn_quantize_fp8); g must be NULL.
 *   FN_UNFUSED: codes and scales of the unfolded W, and g [K] float32; an
 *     RMSNorm kernel writes xn (bf16) to the workspace first (the prefill
 *     path then quantises xn, whose row factor is q alone).
 *   FN_FUSED_PACKED (decode-packed codes) takes M <= 16 only.
 *   FN_TWO_STREAM is not offered.  Errors as fn_norm_linear.
 */
int fn_norm_linear_fp8(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* W8,
                       const float* w_scales, int64_t N, const float* g, float eps, void* y, int y_dtype,
                       int variant, void* ws, size_t ws_bytes, void* stream);

int fn_norm_glu_ffn_fp8(const void* x, int x_dtype, int64_t M, int64_t K, const uint8_t* W8_gate,
                        const float* s_gate, const uint8_t* W8_up, const float* s_up, int64_t N,
                        const float* g, float eps, void* h, int h_dtype, int variant,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * MLA attention input with latent normalisation, the pre-attention RMSNorm
 * dropped by scale invariance (FlashNorm Abstract: this removes the first
 * RMSNorm in MLA models with latent normalisation).  One projection gives
 * the columns [q latent | kv latent | rope part]:
 *   z = x . W*^T            (W* folded with the dropped norm's gain)
 *   q latent  [0, nq):       y = z * g_q  / sqrt(mean over the nq columns of z^2 + eps_latent)
 *   kv latent [nq, nq+nkv):  y = z * g_kv / sqrt(mean over the nkv columns of z^2 + eps_latent)
 *   rope part (n_rope columns, followed by no norm): y = z * s[m],
 *     s[m] = 1/sqrt(mean_k x[m,k]^2 + eps_x), then, when positions are given,
 *     the rotary embedding of fn_linear_qknorm_rope with the part as one head.
 * A latent spans several output tiles, so the GEMM writes the float32
 * product of the latent columns and their 32-column sums of squares to the
 * workspace, and a row kernel applies the latent norms.
 *   n_q_latent, n_kv_latent: multiples of 32 (either may be 0, not both);
 *   n_rope a multiple of 4 (may be 0); W [N x K], N = nq + nkv + n_rope.
 *   g_q_latent [nq], g_kv_latent [nkv] float32 (required for a non-empty
 *   latent).  positions / rope_table / n_pos / rot_dim as in
 *   fn_linear_qknorm_rope, with rot_dim <= n_rope; positions NULL = no
 *   rotation (rope_table ignored).
 *   ws: fn_workspace_bytes(FN_OP_LINEAR_LATENT_NORM, ...) bytes (needed by
 *   both variants).  FN_UNFUSED: unfolded W and g1 [K]; xn = RMSNorm(x; g1,
 *   eps_x) is written first and the rope part is not scaled.  bf16 only.
 */
int fn_linear_latent_norm(const void* x, int x_dtype, int64_t M, int64_t K, const void* W, int w_dtype,
                          int64_t n_q_latent, int64_t n_kv_latent, int64_t n_rope,
                          const float* g_q_latent, const float* g_kv_latent, float eps_x, float eps_latent,
                          const int32_t* positions, const float* rope_table, int64_t n_pos, int rot_dim,
                          const float* g1, void* y, int y_dtype, int variant,
                          void* ws, size_t ws_bytes, void* stream);

/* Release the per-thread events the two-stream variant created. */
void fn_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHNORM_H */
