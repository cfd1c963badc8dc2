/*
 * qmv.h -- fused dequantize-and-multiply of block-quantized weights on
 * AMD Instinct MI355X (gfx950).  C ABI of libqmv.so.
 *
 * What the library computes
 *   y = W x     (decode matvec, a batch of 1..N activation vectors)
 *   Y = X W^T   (prefill GEMM on the matrix cores, small M)
 * directly from packed blocks of small integers with per-block fp16 scales
 * (and mins or zeros), without ever forming the dense W.  The formats are
 * those the pages name: the "packed group-64 W4A16 linear kernels" (llmopt
 * README, "Current compiler and runtime"), Q8_0 and the K-quant Q4_K / Q6_K
 * matvec kernels (aot-llm README, feature list "Static code generation" and
 * "SIMD kernels"), and the Q4_K linear of the llmopt parity receipt
 * ("GGUF-FX parity probe").  The pages give no bit layout or formula; the
 * definitions below are this library's own, and normative.
 *
 * Dequantization (IEEE f32, round to nearest even, in this order, no fusion):
 *   QMV_Q8_0       32-weight blocks:  w = f32(scale) * f32(q),  q int8
 *   QMV_W4A16_G64  64-weight groups:  w = f32(scale) * (f32(q) - f32(zero)),  q in 0..15
 *   QMV_Q4K        256-weight super-blocks of 8 sub-blocks of 32:
 *                  w = (f32(d) * f32(sc_j)) * f32(q) - f32(dmin) * f32(m_j)
 *                  q in 0..15, sc_j and m_j in 0..63
 *   QMV_Q6K        256-weight super-blocks of 16 sub-blocks of 16:
 *                  w = (f32(d) * f32(s_j)) * (f32(q) - 32),  q in 0..63, s_j int8
 *   QMV_Q4_0       32-weight blocks:  w = f32(d) * (f32(q) - 8),   q in 0..15
 *   QMV_Q5_0       32-weight blocks:  w = f32(d) * (f32(q) - 16),  q in 0..31
 *   QMV_Q5K        as QMV_Q4K with q in 0..31
 *   QMV_DENSE_BF16 w = the bf16 value
 *   QMV_I8_ROW     one f32 scale per row:  w = scale_n * f32(q),  q int8
 * The last five are the other weight types the pages' runtimes load: the
 * q4_0, q5_0 and q5_K tensor types of the aot-llm README (and the llmopt
 * README's Q5_0 linear parity receipt), the bf16 resident weights of the
 * zynfer PR's stage M4 and its stage M5 per-row symmetric int8 weights.
 * The scale of weight k is that of block floor(k / block size).  fp16
 * subnormals are honoured.  qmv_dequant reproduces these values bit for bit.
 * qmv_matvec / qmv_gemm may reassociate sums (tolerances below).
 *
 * Logical (unpacked) arrays -- the interchange form taken by qmv_pack,
 * row-major, `batch` matrices stacked back to back:
 *   Q8_0       q int8 [N][K];  aux[0] scale f16 [N][K/32]
 *   W4A16_G64  q uint8 [N][K];  aux[0] scale f16 [N][K/64];  aux[1] zero f16 [N][K/64]
 *   Q4K        q uint8 [N][K];  aux[0] sc uint8 [N][K/32];  aux[1] m uint8 [N][K/32];
 *              aux[2] d f16 [N][K/256];  aux[3] dmin f16 [N][K/256]
 *   Q6K        q uint8 [N][K];  aux[0] s int8 [N][K/16];  aux[1] d f16 [N][K/256]
 *   Q4_0, Q5_0 q uint8 [N][K];  aux[0] d f16 [N][K/32]
 *   Q5K        as Q4K
 *   DENSE_BF16 q bf16 [N][K] (the weights); no aux
 *   I8_ROW     q int8 [N][K];  aux[0] scale f32 [N]
 * Fields wider than their bit width are masked to it by qmv_pack
 * (4 bits for 4-bit q, 5 bits for 5-bit q, 6 bits for Q6K q and for sc / m).
 * K must be a multiple of the format's block: 32, 64 (W4A16_G64) or 256
 * (the K-quants); 32 also for DENSE_BF16 and I8_ROW (the kernels' unit).
 *
 * Packed layout, version 1 (QMV_LAYOUT_VERSION).  One matrix is a sequence
 * of planes; every plane starts at a multiple of 256 bytes (plane sizes are
 * rounded up to 256).  Matrix i of a stack starts at i * qmv_packed_bytes(..,1).
 * Multi-byte fields are little-endian.
 *   Q8_0       qs    N*K bytes:      byte n*K + k = q[n][k]
 *              scale N*(K/32) f16:   element n*(K/32) + b = scale[n][b]
 *   W4A16_G64  qs    N*K/2 bytes:    byte n*K/2 + j = q[n][2j] | q[n][2j+1] << 4
 *              sz    N*(K/64) u32:   word n*(K/64) + g = scale[n][g] | zero[n][g] << 16
 *   Q4K        qs    as W4A16_G64
 *              meta  N*(K/256) 16-byte records; record (n, t): bytes 0-1 d, bytes 2-3
 *                    dmin, bytes 4..15 a 96-bit little-endian integer holding
 *                    sc[n][8t+j] at bits 6j..6j+5 and m[n][8t+j] at bits 48+6j..48+6j+5
 *   Q6K        ql    N*K/2 bytes: low 4 bits of q, nibble order as W4A16_G64
 *              qh    N*(K/16) u32: word (n, t) covers k = 16t..16t+15; its bits
 *                    8c+2f .. 8c+2f+1 (c, f in 0..3) hold bits 4-5 of
 *                    q[n][16t + 8*(f>>1) + 2c + (f&1)]
 *              s     N*(K/16) int8
 *              d     N*(K/256) f16
 *   Q4_0       qs    as W4A16_G64
 *              d     N*(K/32) f16:     element n*(K/32) + b = d[n][b]
 *   Q5_0       qs    as W4A16_G64, low 4 bits of q
 *              qh    N*(K/32) u32: word (n, u) covers k = 32u..32u+31; its bit
 *                    8c + 2i + e (c, i in 0..3, e in 0..1) holds bit 4 of
 *                    q[n][32u + 8i + 2c + e]
 *              d     as Q4_0
 *   Q5K        qs, qh as Q5_0;  meta as Q4K
 *   DENSE_BF16 w     N*K bf16
 *   I8_ROW     qs    N*K bytes;  scale N f32
 * Bytes per weight including scales: Q8_0 8.5 bits, W4A16_G64 4.5, Q4K 4.5, Q6K 6.5625,
 * Q4_0 4.5, Q5_0 5.5, Q5K 5.5, DENSE_BF16 16, I8_ROW 8 + 32/K.
 *
 * Accuracy of the products.  For every output,
 *   |y - y_exact| <= tau * ||W_row||_2 * ||x||_2
 * with tau = 1e-3 for qmv_matvec (f32 accumulation) and tau = 2e-2 for
 * qmv_gemm (bf16 matrix-core inputs, bf16 output).  With a one-hot x the
 * matvec returns the dequantized column bit for bit.
 *
 * Ownership and threading.  The caller allocates and owns every buffer; all
 * pointers passed to compute calls are device pointers.  The compute calls
 * never allocate, free, synchronize or copy between host and device; they
 * enqueue kernels on `stream` (a hipStream_t; NULL = the null stream) and
 * return at once, so they may be captured in a hipGraph.  The library keeps
 * no state but a per-device architecture check; calls are thread-safe.
 *
 * Errors.  Every call returns QMV_OK (0) or a negative qmv_status.  All
 * argument errors are found on the host before anything is enqueued; the
 * thread-local qmv_last_error() then names the argument.  QMV_ERR_LAUNCH
 * reports a failed launch; faults during execution surface at the caller's
 * next synchronization, as usual for HIP.
 */
#ifndef QMV_H_
#define QMV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMV_ABI_VERSION 3
#define QMV_LAYOUT_VERSION 1

enum qmv_format {
  QMV_Q8_0 = 1,
  QMV_W4A16_G64 = 2,
  QMV_Q4K = 3,
  QMV_Q6K = 4,
  QMV_Q4_0 = 5,
  QMV_Q5_0 = 6,
  QMV_Q5K = 7,
  QMV_DENSE_BF16 = 8,
  QMV_I8_ROW = 9
};

enum qmv_dtype {
  QMV_F32 = 1,
  QMV_F16 = 2,
  QMV_BF16 = 3,
  QMV_Q8X = 4  /* activations quantized to 8-bit blocks by qmv_quantize_x (layout below) */
};

enum qmv_status {
  QMV_OK = 0,
  QMV_ERR_NULL = -1,        /* a required pointer is NULL */
  QMV_ERR_FORMAT = -2,      /* unknown format value */
  QMV_ERR_UNSUPPORTED = -3, /* valid but not implemented (format / dtype / op) */
  QMV_ERR_SHAPE = -4,       /* N < 1, K < 1, K not a multiple of the block, batch < 1 */
  QMV_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
  QMV_ERR_DTYPE = -6,       /* unknown dtype value */
  QMV_ERR_OVERFLOW = -7,    /* a size does not fit in size_t / int32 indexing */
  QMV_ERR_DEVICE = -8,      /* current device is not gfx950 or HIP query failed */
  QMV_ERR_LAUNCH = -9       /* hipGetLastError after the launch */
};

/* Per-format logical arrays for qmv_pack (device pointers); see above. */
typedef struct qmv_logical {
  const void* q;
  const void* aux[4];
} qmv_logical;

/* One matrix of a grouped matvec (all pointers are device pointers). */
typedef struct qmv_matvec_item {
  int64_t N;     /* rows of this matrix */
  const void* W; /* packed matrix, layout above, 16-byte aligned */
  const void* x; /* [batch][K] activations; items may share one x */
  void* y;       /* [batch][N] output; must not overlap another item's y */
  int32_t fmt;   /* this matrix's qmv_format, or 0 for the call's fmt */
} qmv_matvec_item;

/*
 * ABI version (QMV_ABI_VERSION); *layout_version receives QMV_LAYOUT_VERSION
 * if non-NULL.  Host only, never fails.  A caller that links the library as a
 * C library (aot-llm README, compiler options: a model built as a static or
 * shared library with a C API and a symbol prefix) checks both numbers
 * before it hands over buffers packed by another build.
 */
int qmv_abi_version(int* layout_version);

/*
 * Static text for a status code ("unknown status" for a value outside
 * qmv_status).  Host only; the string is never freed.  Status codes and the
 * message below are how unsupported requests are rejected before any work is
 * queued, naming what is missing (aot-llm README, supported tensor types:
 * unsupported types are rejected with a message naming the tensor;
 * pytensor-ml issue 53, PR 6 item F-28: unsupported combinations fail before
 * the first token).
 */
const char* qmv_status_string(int status);

/*
 * Thread-local message of the last failing call on this thread ("" after a
 * call that succeeded); it names the argument, item or capability at fault
 * (same passages as qmv_status_string).  Valid until the next call on the
 * same thread.
 */
const char* qmv_last_error(void);

/*
 * Bytes of `batch` stacked packed matrices of shape N x K.  Host only.  Every
 * product is checked for overflow before it is formed, and K must be a whole
 * number of blocks (pytensor-ml issue 53, PR 15 item F-39: checked block and
 * tail arithmetic for packed tensors).
 * Errors: FORMAT, SHAPE, NULL (out_bytes), OVERFLOW.
 */
int qmv_packed_bytes(int fmt, int64_t N, int64_t K, int64_t batch, size_t* out_bytes);

/*
 * Pack `batch` stacked logical matrices (device arrays as listed above) into
 * dst (device, qmv_packed_bytes bytes, 256-byte aligned recommended, 16
 * required).  Integer bit placement only (pytensor-ml issue 53, PR 17: a
 * one-time repack, done once per matrix outside the token loop).
 * Errors: FORMAT, SHAPE, NULL, ALIGN, OVERFLOW, DEVICE, LAUNCH.
 */
int qmv_pack(int fmt, int64_t N, int64_t K, int64_t batch, const qmv_logical* src,
             void* dst, void* stream);

/*
 * y[b][n] = sum_k W[n][k] * x[b][k] for b < batch, n < N.
 *   W  packed matrix (device), layout above
 *   x  [batch][K] of x_dtype (QMV_F32 or QMV_F16), device, 16-byte aligned
 *   y  [batch][N] of y_dtype (QMV_F32), device, 4-byte aligned
 * The decode matvec of the pages' runtimes (aot-llm README, Metal backend
 * notes: matrix-vector kernels with f32 activations and weights dequantized
 * on the fly; batched prompt notes: each weight decoded once for several
 * activations).  Any batch >= 1 is accepted; up to 8 vectors share one pass
 * over W.  x_dtype QMV_F16 is taken by QMV_W4A16_G64 only.
 * Errors: FORMAT, SHAPE, NULL, ALIGN, DTYPE, UNSUPPORTED, OVERFLOW, DEVICE, LAUNCH.
 */
int qmv_matvec(int fmt, int64_t N, int64_t K, int64_t batch, const void* W,
               const void* x, int x_dtype, void* y, int y_dtype, void* stream);

/* Fused epilogue of qmv_matvec_ex (all device pointers, f32, 4-byte aligned). */
typedef struct qmv_epilogue {
  const float* bias;      /* [N] added to every vector's product, or NULL */
  const float* residual;  /* [batch][N] added last, or NULL; may be y itself (y += W x) but
                             must not otherwise overlap y */
} qmv_epilogue;

/*
 * y[b][n] = residual[b][n] + (sum_k W[n][k] * x[b][k] + bias[n]), the bias and
 * residual adds fused into the matvec's epilogue (aot-llm README, Metal
 * backend notes: the q / k / v kernels add their biases in the epilogue, wo
 * and down fuse the residual add).  ep == NULL, or both pointers NULL, is
 * qmv_matvec.  Arguments otherwise as qmv_matvec.  The epilogue adds two f32
 * roundings to the matvec tolerance.  Batch 2..8 with an epilogue runs on the
 * FMA kernel (the matrix-core kernel has none).
 * Errors: as qmv_matvec, plus ALIGN for a misaligned bias / residual.
 */
int qmv_matvec_ex(int fmt, int64_t N, int64_t K, int64_t batch, const void* W, const void* x, int x_dtype,
                  void* y, int y_dtype, const qmv_epilogue* ep, void* stream);

/*
 * h[b][n] = silu(g) * u with g = sum_k Wg[n][k] x[b][k], u = sum_k Wu[n][k] x[b][k]
 * and silu(z) = z / (1 + exp(-z)): the gate / up projections and the SwiGLU
 * product in one pass (aot-llm README, Metal backend notes: the fused
 * gate / up / SwiGLU product).  W_gate and W_up are packed matrices of the
 * same format and shape; each row of both is read once, and only h is
 * written.  x, h and dtypes as qmv_matvec (h is y).  Tolerance: the matvec
 * bound of g and u propagated through silu (Lipschitz 1.1) and the product.
 * Errors: as qmv_matvec (NULL names W_gate or W_up).
 */
int qmv_matvec_swiglu(int fmt, int64_t N, int64_t K, int64_t batch, const void* W_gate, const void* W_up,
                      const void* x, int x_dtype, void* h, int h_dtype, void* stream);

/*
 * Several matvecs of one K and one batch in as few launches as possible: for
 * every item i, y_i[b][n] = sum_k W_i[n][k] * x_i[b][k].
 * The grouped dispatch of the pages' decoders: the q / k / v projections in
 * one dispatch with the simdgroups spread over the three matrices, gate / up
 * in another (aot-llm README, Metal backend notes).  An item's format is its
 * own fmt field, or the call's `fmt` where that field is 0 (`fmt` may be 0
 * only if every item names its own).  Up to 16 items share one launch (per
 * chunk of 8 vectors at batch >= 2); the launch's workgroups are split over
 * the items in proportion to their rows.  Q4K and Q6K items may share a
 * launch (a layer whose v projection is Q6K next to Q4K q and k); other mixes
 * run one launch series per format.  Items outside the grouped kernels' range
 * (K above 6144 at batch >= 2, or an activation slice too wide for registers
 * at batch 1) run one qmv_matvec launch each.  Each item's result equals its
 * qmv_matvec result bit for bit, with one exception: at batch 1 with
 * 512 < K <= 1024, a launch of more than 16384 rows in all gives each row 16
 * lanes instead of 32, so an item whose single call falls on the other side
 * of that size is summed in another order (both within the matvec
 * tolerance).  Dtypes and alignment as qmv_matvec (x_dtype
 * must suit every item's format); 1 <= count <= 4096.
 * Errors: FORMAT, SHAPE, NULL, ALIGN, DTYPE, UNSUPPORTED, OVERFLOW, DEVICE, LAUNCH
 * (the message names the offending item).
 */
int qmv_matvec_grouped(int fmt, int64_t K, int64_t batch, int count, const qmv_matvec_item* items,
                       int x_dtype, int y_dtype, void* stream);

/*
 * Y[m][n] = sum_k X[m][k] * W[n][k] for m < M, on bf16 matrix cores with f32
 * accumulation; each weight is dequantized once per token tile, in registers,
 * straight into the matrix-core operand (aot-llm README, Metal backend notes:
 * prompt batches use a tiled GEMM on the matrix units with the weights
 * dequantized once per tile).
 *   fmt   QMV_W4A16_G64 (others -> UNSUPPORTED)
 *   X     [M][K] of x_dtype QMV_BF16, device, 16-byte aligned
 *   Y     [M][N] of y_dtype QMV_BF16, device, 4-byte aligned
 * Errors: FORMAT, SHAPE, NULL, ALIGN, DTYPE, UNSUPPORTED, OVERFLOW, DEVICE, LAUNCH.
 */
int qmv_gemm(int fmt, int64_t N, int64_t K, int64_t M, const void* W, const void* X,
             int x_dtype, void* Y, int y_dtype, void* stream);

/*
 * Quantize `batch` f32 activation vectors x [batch][K] (K a multiple of 32) to
 * 8-bit blocks, once, for the integer-dot matvec: per vector and block of 32,
 *   amax = max |x_k|,  d = amax / 127,  id = 127 / amax,
 *   q_k = rint(x_k * id) clamped to [-127, 127]   (f32 operations, round to
 *   nearest even; the quantized activation is d * q_k),
 * except that a block with amax < 2^-120 (where 127 / amax could overflow)
 * gets d = 0 and zero codes.  x must be finite (otherwise the codes are
 * unspecified)
 * (aot-llm README, How it works: per matmul the f32 activation vector is
 * quantized once to 8-bit blocks and every output row is an integer dot
 * product scaled back to f32).  xq receives, per vector b at byte
 * b * R with R = (K + K/8) rounded up to 16: K int8 codes, then K/32 f32
 * scales d; qmv_q8x_bytes gives the size.  Codes and scales are unique bit
 * for bit.  Pass xq to qmv_matvec / qmv_matvec_ex / qmv_matvec_swiglu /
 * qmv_matvec_grouped with x_dtype QMV_Q8X: the formats Q8_0, W4A16_G64, Q4K,
 * Q6K, Q4_0, Q5_0, Q5K and I8_ROW then take integer dot products (exact in
 * int32) per 32-weight block, scaled back in f32.  The result matches the
 * product over d * q within the matvec tolerance; against the f32 x it also
 * carries the quantization error (|x - d q| <= d / 2 per element, about
 * 5e-3 relative for N(0,1) activations).
 * Errors: SHAPE (K not a multiple of 32, batch < 1), NULL, ALIGN (16 bytes),
 * OVERFLOW, DEVICE, LAUNCH.
 */
int qmv_quantize_x(int64_t K, int64_t batch, const float* x, void* xq, void* stream);

/* Bytes of the qmv_quantize_x output for `batch` vectors of K.  Host only.
 * Errors: SHAPE, NULL, OVERFLOW. */
int qmv_q8x_bytes(int64_t K, int64_t batch, size_t* out_bytes);

/*
 * Dense f32 dequantization of one packed matrix into out [N][K] (device),
 * bit-exact to the definitions above (the correctness baseline's dense
 * conversion, pytensor-ml issue 53, PR 15 item F-41).  A test/inspection
 * export: the hot path never calls it.
 * Errors: FORMAT, SHAPE, NULL, ALIGN, OVERFLOW, DEVICE, LAUNCH.
 */
int qmv_dequant(int fmt, int64_t N, int64_t K, const void* W, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H_ */
