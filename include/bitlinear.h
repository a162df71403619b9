/*
 * bitlinear.h - C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear library.
 *
 * The library computes the ternary-weight / int8-activation projection
 *
 *     Y = (X~ W~^T) * gamma * beta / 127
 *
 * defined on the page "BitNet b1.58: Mathematical Foundations of 1.58-Bit
 * Ternary Quantization, Absmean Scaling, and Multiplication-Free LLM
 * Architectures" (llms.blog), section 2 "Mathematical Formulation of the
 * BitLinear b1.58 Layer": the absmean weight quantiser, the absmax activation
 * quantiser, and the linear transformation with its rescale.  The integer
 * product X~ W~^T uses only additions and subtractions of int8 values into
 * int32 (same section, last paragraph; section 6 "Vectorized Ternary GEMV
 * with SIMD" gives the masked-add form).
 *
 * Conventions for every entry point
 *   - Shapes: N = d_out (rows of W), K = d_in, M = tokens.  W is [N][K]
 *     row-major fp32, X is [M][K] row-major fp32, Y is [M][N] row-major.
 *   - All buffers are device memory allocated and owned by the caller.  The
 *     library never allocates, never frees, and keeps no pointer after a
 *     call returns.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream of the current device).  Buffers must stay valid
 *     until that work completes.  Calls are stateless and re-entrant; the same
 *     inputs give the same output bytes on every call.
 *   - Arguments are validated before any HIP call; an invalid call returns a
 *     status without touching the GPU.  A launch failure returns
 *     BITLINEAR_ERR_HIP.  Faults during execution surface at the caller's
 *     next synchronisation.  bitlinear_last_error() gives a thread-local
 *     description of the last non-OK status.
 *   - Inputs must be finite; NaN or infinity give unspecified (but memory
 *     safe) results.
 *   - Limits: K % 16 == 0; 1 <= K <= 131072 (so |acc| < 2^24 and the int32
 *     accumulator converts to fp32 exactly); N*K < 2^31 for packing.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_ABI_VERSION 1
/* Packed weight format: 2 bits per weight, see bitlinear_pack_weights. */
#define BITLINEAR_PACK_FORMAT_BLT2_V1 1
#define BITLINEAR_MAX_K 131072
/* Projections per grouped call (bitlinear_forward_grouped). */
#define BITLINEAR_MAX_GROUP 4

typedef enum bitlinear_status {
  BITLINEAR_OK = 0,
  BITLINEAR_ERR_NULL = 1,      /* a required pointer is NULL */
  BITLINEAR_ERR_SHAPE = 2,     /* M, N or K < 1, K % 16 != 0, K > BITLINEAR_MAX_K, size limit */
  BITLINEAR_ERR_ALIGN = 3,     /* a pointer is not aligned as documented */
  BITLINEAR_ERR_DTYPE = 4,     /* unknown output dtype */
  BITLINEAR_ERR_NO_DEVICE = 5, /* no HIP device visible */
  BITLINEAR_ERR_ARCH = 6,      /* current device is not gfx950 */
  BITLINEAR_ERR_WORKSPACE = 7, /* workspace NULL or smaller than the size query */
  BITLINEAR_ERR_HIP = 8        /* a HIP runtime call or kernel launch failed */
} bitlinear_status;

typedef enum bitlinear_dtype {
  BITLINEAR_F32 = 0,  /* fp32 Y */
  BITLINEAR_BF16 = 1, /* bf16 Y, rounded to nearest even from the fp32 result */
  BITLINEAR_I32 = 2   /* raw int32 accumulators X~ W~^T, no rescale */
} bitlinear_dtype;

/* Version of this ABI (BITLINEAR_ABI_VERSION). */
int bitlinear_abi_version(void);

/* Bytes of packed weights for an N x K matrix: N * K / 4.  0 if the shape is
 * invalid. */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);

/* Bytes of workspace bitlinear_pack_weights needs for an N x K matrix
 * (partial sums of the exact |W| accumulator and the two ternary
 * thresholds).  0 if the shape is invalid. */
size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K);

/*
 * Absmean ternarisation and 2-bit packing of a latent weight matrix.
 * Page section 2, "Weight Quantization: Absmean Scaling":
 *   gamma = mean_ij |W_ij|,   W~_ij = RoundClip(W_ij / (gamma + eps), -1, 1),
 *   RoundClip(z, a, b) = max(a, min(b, floor(z + 0.5))),  eps = 1e-5.
 *
 * gamma is the exact mean of |W| rounded once to fp32 (nearest, ties to
 * even); gamma + eps is an fp32 addition; z = W / (gamma + eps) is the
 * correctly rounded fp32 quotient and floor(z + 0.5) is taken exactly.
 *
 * W          [N][K] fp32, device, 16-byte aligned (read only).
 * W_packed   [N][K/4] bytes, device, 16-byte aligned (written).  Format
 *            BLT2-v1: code c = W~ + 1 in {0,1,2} (3 never occurs).  Row n is
 *            K/16 little-endian 32-bit words at byte n*K/4; word g holds
 *            k = 16g + t, t = 0..15, and weight t = 4j + i sits in byte i at
 *            bits 2j..2j+1.  So (word >> 2j) & 0x03030303 holds the codes of
 *            k = 16g+4j .. 16g+4j+3 in byte order.  An all-zero group is
 *            0x55555555.
 * gamma      one fp32, device, 4-byte aligned (written): the absmean scale.
 * workspace  device, 16-byte aligned, >= bitlinear_pack_workspace_bytes(N, K).
 *            Contents need no initialisation and are scratch after the call.
 * stream     hipStream_t or NULL.
 */
bitlinear_status bitlinear_pack_weights(const float* W, int64_t N, int64_t K,
                                        uint8_t* W_packed, float* gamma,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Per-token absmax int8 quantisation of activations.  Page section 2,
 * "Activation Quantization: Absmax Scaling" (per-token variant, symmetric
 * range, Q_b - 1 = 127):
 *   beta_m = max_k |X_mk|,
 *   X~_mk = RoundClip(X_mk * (127 / (beta_m + eps)), -127, 127).
 * The factor 127 / (beta_m + eps) is formed in fp32 (add, then correctly
 * rounded divide), each element is multiplied by it in fp32, and
 * floor(q + 0.5) is taken exactly.
 *
 * X        [M][K] fp32, device, 16-byte aligned (read only).
 * X_q      [M][K] int8, device, 16-byte aligned (written).
 * x_scale  [M] fp32, device, 4-byte aligned (written): beta_m / 127 rounded
 *          to fp32 (the per-token factor of the rescale).
 * x_sum    [M] int32, device, 4-byte aligned (written): sum_k X~_mk.  The
 *          forward pass needs it (it stores W~ + 1 and subtracts this sum).
 */
bitlinear_status bitlinear_quant_acts(const float* X, int64_t M, int64_t K,
                                      int8_t* X_q, float* x_scale, int32_t* x_sum,
                                      void* stream);

/*
 * The quantiser of bitlinear_quant_acts at b-bit width (page section 2,
 * absmax scaling with Q_b = 2^(b-1) levels per sign): bits = 8 computes
 * exactly bitlinear_quant_acts; bits = 4 gives the 4-bit activations ("A4")
 * of the W1A4KV2 combination that the page "The End of Matrix
 * Multiplications: Welcome to Addition" names without a quantiser:
 *   X~ = RoundClip(X * 7 / (beta + eps), -7, 7),  x_scale = beta / 7,
 * stored one value per int8 element, so every projection entry point
 * (bitlinear_forward, _grouped, _base3) takes them unchanged and its
 * epilogue rescales by that x_scale.  Arguments as bitlinear_quant_acts;
 * bits other than 8 and 4 return BITLINEAR_ERR_DTYPE.
 */
bitlinear_status bitlinear_quant_acts_bits(const float* X, int64_t M, int64_t K, int bits,
                                           int8_t* X_q, float* x_scale, int32_t* x_sum,
                                           void* stream);

/* Bytes of workspace bitlinear_forward needs: int32 partial accumulators
 * where K is split across workgroups (added exactly by a second launch):
 * the tiled product with few output tiles and a long K (e.g. 65 <= M <= 128
 * with M K > 256 Ki, or 33 <= M <= 64 with K > 8192, on a few-thousand-row
 * matrix), and the skinny kernel on a K at least twice N at 17 <= M <= 64
 * with M K > 256 Ki; else 0 (a NULL
 * workspace is then accepted).  0 if the shape is invalid. */
size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * The projection on packed weights and quantised activations.  Page section
 * 2, "The Linear Transformation and Rescaling":
 *   acc[m][n] = sum_k W~[n][k] X~[m][k]        (exact, int32)
 *   Y[m][n]   = acc[m][n] * gamma * x_scale[m]  (fp32: (float)acc * gamma,
 *               then * x_scale; bf16 rounds that fp32 value to nearest even)
 * The scale is applied once per output after the integer sum (page section
 * 6, "Scaling Factor Fusion").
 *
 * W_packed  [N][K/4] BLT2-v1 bytes from bitlinear_pack_weights, device,
 *           16-byte aligned.
 * gamma     one fp32, device.
 * X_q, x_scale, x_sum   as written by bitlinear_quant_acts (device; X_q
 *           16-byte aligned).  x_sum must equal sum_k X_q[m][k].
 * Y         [M][N], device, aligned to its element size; fp32, bf16 or int32
 *           (BITLINEAR_I32 stores acc itself and ignores gamma/x_scale).
 * workspace device, 16-byte aligned, >= bitlinear_forward_workspace_bytes(M,
 *           N, K) bytes; contents need no initialisation and are scratch after
 *           the call (two calls in flight at once need two workspaces).  May
 *           be NULL when the size query returns 0.
 * Integer results are bit-exact and independent of the launch shape (split
 * partial sums are added in exact int32 arithmetic).  Which kernel runs
 * (bitlinear_forward_kernel reports it) depends only on M, N and K.
 */
bitlinear_status bitlinear_forward(const uint8_t* W_packed, const float* gamma,
                                   int64_t N, int64_t K,
                                   const int8_t* X_q, const float* x_scale,
                                   const int32_t* x_sum, int64_t M,
                                   void* Y, bitlinear_dtype y_dtype,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Bytes of workspace bitlinear_forward_f32 needs: 0 when the shape runs as
 * one fused launch, else room for X~, x_scale and x_sum followed by the
 * projection's own workspace (bitlinear_forward_workspace_bytes).  0 if the
 * shape is invalid. */
size_t bitlinear_forward_f32_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Activation quantisation fused with the projection: fp32 X in, Y out.
 * Computes exactly bitlinear_quant_acts followed by bitlinear_forward (same
 * X~, same x_scale, same x_sum, same accumulators; page section 2, absmax
 * activation quantiser and the linear transformation), as one launch for
 * single-token shapes (K a multiple of 64 up to 16384, or longer rows whose
 * int8 copy fits the on-chip staging; one projection of 2^25 weights or
 * more, with K a multiple of 64 up to 32768, takes the persistent launch of
 * bitlinear_forward_f32_multi)
 * and two-token narrow ones (every workgroup quantises the activations it
 * needs), else as those two launches.  This is the quantiser folded into
 * the projection's prologue.
 *
 * X        [M][K] fp32, device, 16-byte aligned (read only).
 * Y        [M][N], device, as in bitlinear_forward.
 * X_q_out, x_scale_out, x_sum_out  optional (all three or none): receive the
 *          quantiser outputs, as bitlinear_quant_acts would write them.
 * workspace  bitlinear_forward_f32_workspace_bytes(M, N, K) bytes (16-byte
 *          aligned), scratch after the call.  May be NULL when that is 0, or
 *          when the outputs are given and bitlinear_forward_workspace_bytes
 *          (M, N, K) is 0.
 */
bitlinear_status bitlinear_forward_f32(const uint8_t* W_packed, const float* gamma,
                                       int64_t N, int64_t K, const float* X, int64_t M,
                                       void* Y, bitlinear_dtype y_dtype,
                                       int8_t* X_q_out, float* x_scale_out, int32_t* x_sum_out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * bitlinear_forward_f32 for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same computation and results, byte for byte, as
 * bitlinear_forward_f32 with the same arguments; the workspace is not the
 * caller's but a fixed array of BITLINEAR_NOALLOC_SCRATCH_BYTES in device
 * memory that the library holds on each GPU it runs on, reserved when its code
 * loads on that device and kept until the process ends.  The call allocates
 * and frees nothing.  The caller still owns X, Y and the optional quantiser
 * outputs (as in bitlinear_forward_f32).
 *
 * Every call on one GPU shares that GPU's array: two calls that overlap in
 * time on one GPU (different streams or host threads) race on it and give
 * unspecified results; calls in order on one stream are safe.  Nothing in the
 * array needs clearing between calls.
 * Errors as bitlinear_forward_f32, and BITLINEAR_ERR_WORKSPACE (before any HIP
 * call) when bitlinear_forward_f32_workspace_bytes(M, N, K) exceeds
 * BITLINEAR_NOALLOC_SCRATCH_BYTES (long-K prefill shapes with many tokens).
 */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES (32u << 20)
bitlinear_status bitlinear_forward_f32_noalloc(const uint8_t* W_packed, const float* gamma,
                                               int64_t N, int64_t K, const float* X, int64_t M,
                                               void* Y, bitlinear_dtype y_dtype, int8_t* X_q_out,
                                               float* x_scale_out, int32_t* x_sum_out,
                                               void* stream);

/*
 * Several projections of one activation matrix in one call: the query, key
 * and value projections of an attention block, or the gate and up
 * projections of a feed-forward block, which all read the same X~.  For
 * g < G this computes exactly what bitlinear_forward(W_packed[g], gamma[g],
 * N[g], K, X_q, x_scale, x_sum, M, Y[g], y_dtype, ...) computes (page
 * section 2, "The Linear Transformation and Rescaling").  Decode shapes
 * (M <= 16, and up to 64 tokens where the skinny kernel applies) run as one
 * launch over the rows of all G matrices, so the group pays one launch
 * instead of G; tiled-product shapes run the projections one after another.
 * With G > 1 the skinny kernel never splits K (with G = 1 the call is
 * bitlinear_forward, which may).
 *
 * G          1 .. BITLINEAR_MAX_GROUP.
 * W_packed, gamma, N, Y   HOST arrays of G entries (read during the call,
 *            not kept); the buffers they point to are device memory, laid
 *            out and aligned as for bitlinear_forward.  All projections share
 *            K, M, X_q, x_scale and x_sum.
 * workspace  >= bitlinear_forward_grouped_workspace_bytes(M, G, N, K) bytes
 *            (16-byte aligned), scratch after the call; may be NULL when that
 *            is 0 (it is 0 for M <= 16).
 */
size_t bitlinear_forward_grouped_workspace_bytes(int64_t M, int G, const int64_t* N, int64_t K);
bitlinear_status bitlinear_forward_grouped(int G, const uint8_t* const* W_packed,
                                           const float* const* gamma, const int64_t* N,
                                           int64_t K, const int8_t* X_q, const float* x_scale,
                                           const int32_t* x_sum, int64_t M, void* const* Y,
                                           bitlinear_dtype y_dtype, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * The grouped projection from fp32 activations: X is quantised once (page
 * section 2, absmax activation quantiser), then every projection as in
 * bitlinear_forward_grouped; for decode shapes whose rows in total fit the
 * fused kernel this is a single launch.  Arguments as in
 * bitlinear_forward_f32, with the per-projection arrays as in
 * bitlinear_forward_grouped.
 *
 * workspace  bitlinear_forward_f32_grouped_workspace_bytes(M, G, N, K) bytes
 *            (16-byte aligned), scratch after the call.  May be NULL when
 *            that is 0, or when the quantiser outputs are given and
 *            bitlinear_forward_grouped_workspace_bytes(M, G, N, K) is 0.
 */
size_t bitlinear_forward_f32_grouped_workspace_bytes(int64_t M, int G, const int64_t* N,
                                                     int64_t K);
bitlinear_status bitlinear_forward_f32_grouped(int G, const uint8_t* const* W_packed,
                                               const float* const* gamma, const int64_t* N,
                                               int64_t K, const float* X, int64_t M,
                                               void* const* Y, bitlinear_dtype y_dtype,
                                               int8_t* X_q_out, float* x_scale_out,
                                               int32_t* x_sum_out, void* workspace,
                                               size_t workspace_bytes, void* stream);

/*
 * Several projections, each with its own activations and its own K, in one
 * call: the projections of a decode step that do not share an input (two
 * feed-forward projections on separate inputs, the experts of a
 * mixture-of-experts layer with their own tokens).  For g < G this computes
 * exactly what bitlinear_forward_f32(W_packed[g], gamma[g], N[g], K[g], X[g],
 * M, Y[g], y_dtype, ...) computes (page section 2, absmax activation
 * quantiser and the linear transformation; same X~, accumulators and output
 * bytes).  One token (M = 1) with every K[g] a multiple of 64 up to 32768
 * runs as ONE launch that streams the weights of all G matrices (page section
 * 4: decode time is the time to read the weights, so the projections share
 * one pass instead of paying a launch each): each workgroup quantises its
 * projection's X once and reads its share of the rows.  Other shapes run the
 * projections one after another; where none of them has a single-launch
 * fused path (more than two tokens, or rows past the fused kernels' reach),
 * all G inputs are quantised by ONE launch first (the same per-row
 * arithmetic, into the workspace), then each projection is one launch.
 *
 * G          1 .. BITLINEAR_MAX_GROUP.
 * W_packed, gamma, N, K, X, Y   HOST arrays of G entries (read during the call,
 *            not kept); the buffers are device memory laid out and aligned as
 *            for bitlinear_forward_f32 (X[g] is [M][K[g]] fp32, 16-byte
 *            aligned; W_packed[g] is [N[g]][K[g]/4] BLT2-v1 bytes).
 * workspace  >= bitlinear_forward_f32_multi_workspace_bytes(M, G, N, K) bytes
 *            (16-byte aligned), scratch after the call; may be NULL when that is
 *            0 (it is 0 for the single launch, and for single-token calls that
 *            fall back to one call per projection).  With the shared quantiser
 *            launch it holds every input's X~, scales and sums (each region
 *            rounded up to 256 bytes) and then the largest projection
 *            workspace.
 * bitlinear_forward_f32_multi_kernel tells which way a call runs.
 */
size_t bitlinear_forward_f32_multi_workspace_bytes(int64_t M, int G, const int64_t* N,
                                                   const int64_t* K);
bitlinear_status bitlinear_forward_f32_multi(int G, const uint8_t* const* W_packed,
                                             const float* const* gamma, const int64_t* N,
                                             const int64_t* K, const float* const* X, int64_t M,
                                             void* const* Y, bitlinear_dtype y_dtype,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream);

/*
 * RMS normalisation before the quantiser.  Page section 2 (activations are
 * normalised with RMSNorm before they are quantised to int8; the page cites
 * Zhang and Sennrich, "Root Mean Square Layer Normalization"):
 *   y_k = x_k / sqrt(mean_k x_k^2 + eps) * g_k,   eps = 1e-5,
 * per token, with a gain vector g and no centring.  The mean of squares is
 * the exact rational sum_k x_k^2 / K rounded once to fp32 (nearest, ties to
 * even; the sum is accumulated in exact integer arithmetic, so the result does
 * not depend on the launch shape); then one fp32 add, a correctly rounded fp32
 * square root and reciprocal r, and y_k = fl32(fl32(x_k r) g_k).  Then y goes
 * through exactly bitlinear_quant_acts.
 *
 * X       [M][K] fp32, device, 16-byte aligned (read only).
 * norm_g  [K] fp32 gain, device, 16-byte aligned (read only).
 * X_q, x_scale, x_sum   as in bitlinear_quant_acts.
 * Errors as in bitlinear_quant_acts (a NULL gain is BITLINEAR_ERR_NULL).
 */
bitlinear_status bitlinear_rmsnorm_quant(const float* X, const float* norm_g, int64_t M,
                                         int64_t K, int8_t* X_q, float* x_scale, int32_t* x_sum,
                                         void* stream);

/* Bytes of workspace bitlinear_forward_rmsnorm needs (the rules of
 * bitlinear_forward_f32_workspace_bytes; normalisation is fused only into the
 * single-token launch, so some multi-token shapes that fuse in
 * bitlinear_forward_f32 take two launches here).  0 if the shape is invalid. */
size_t bitlinear_forward_rmsnorm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * RMS normalisation, quantiser and projection: bitlinear_rmsnorm_quant
 * followed by bitlinear_forward (same X~, x_scale, x_sum and accumulators).
 * One launch for one token with K a multiple of 64 up to 12288 (the fp32 row
 * and the gain are held in registers while the sum of squares forms), else
 * those two launches.  Arguments as in bitlinear_forward_f32, plus the gain norm_g
 * ([K] fp32, device, 16-byte aligned); workspace from
 * bitlinear_forward_rmsnorm_workspace_bytes, with the same exception when the
 * quantiser outputs are given.
 */
bitlinear_status bitlinear_forward_rmsnorm(const uint8_t* W_packed, const float* gamma, int64_t N,
                                           int64_t K, const float* X, const float* norm_g,
                                           int64_t M, void* Y, bitlinear_dtype y_dtype,
                                           int8_t* X_q_out, float* x_scale_out,
                                           int32_t* x_sum_out, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* The grouped form (up to BITLINEAR_MAX_GROUP projections of one normalised
 * activation matrix, arrays as in bitlinear_forward_grouped): the usual place
 * of the normalisation, in front of the q/k/v or up/gate projections. */
size_t bitlinear_forward_rmsnorm_grouped_workspace_bytes(int64_t M, int G, const int64_t* N,
                                                         int64_t K);
bitlinear_status bitlinear_forward_rmsnorm_grouped(int G, const uint8_t* const* W_packed,
                                                   const float* const* gamma, const int64_t* N,
                                                   int64_t K, const float* X,
                                                   const float* norm_g, int64_t M,
                                                   void* const* Y, bitlinear_dtype y_dtype,
                                                   int8_t* X_q_out, float* x_scale_out,
                                                   int32_t* x_sum_out, void* workspace,
                                                   size_t workspace_bytes, void* stream);

/*
 * Base-3 weights, format BLT3-v1: five ternary weights per byte, 1.6 bits
 * per weight.  Page section 4, "Memory Bandwidth and Latency Bounds": five
 * ternary values fit one byte because 3^5 = 243 < 256.  The layout is this
 * library's own: code c = W~ + 1; a row is padded with W~ = 0 to a multiple
 * of 80 weights and takes 16 * ceil(K / 80) bytes; little-endian 32-bit word
 * g of a row holds k = 20g + 4j + b (j = 0..4, b = 0..3) in its byte b, which
 * stores Nb = sum_j c_{20g+4j+b} 3^(4-j) as ceil(256 Nb / 243).  Same gamma
 * and the same ternary codes as bitlinear_pack_weights; only the packing
 * differs.
 */
#define BITLINEAR_PACK_FORMAT_BLT3_V1 2
/* Tokens per bitlinear_forward_base3 call. */
#define BITLINEAR_BASE3_MAX_M 16

/* Bytes of BLT3-v1 weights for an N x K matrix: N * 16 * ceil(K / 80).  0 if
 * the shape is invalid (as for bitlinear_packed_bytes). */
size_t bitlinear_packed3_bytes(int64_t N, int64_t K);

/*
 * Absmean ternarisation (as bitlinear_pack_weights: page section 2, "Weight
 * Quantization: Absmean Scaling"; gamma bit for bit the same) packed as
 * BLT3-v1.
 *
 * W          [N][K] fp32, device, 16-byte aligned (read only).
 * W_packed3  bitlinear_packed3_bytes(N, K) bytes, device, 16-byte aligned
 *            (written).
 * gamma      one fp32, device, 4-byte aligned (written).
 * workspace  device, 16-byte aligned, >= bitlinear_pack_workspace_bytes(N, K)
 *            bytes, scratch after the call.
 * Errors as bitlinear_pack_weights.
 */
bitlinear_status bitlinear_pack_weights_base3(const float* W, int64_t N, int64_t K,
                                              uint8_t* W_packed3, float* gamma,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream);

/*
 * The projection of bitlinear_forward (page section 2, "The Linear
 * Transformation and Rescaling"; same accumulators, same epilogue) on BLT3-v1
 * weights, for 1 <= M <= BITLINEAR_BASE3_MAX_M tokens (decode).  Larger M:
 * convert the weights once with bitlinear_base3_to_blt2 and call
 * bitlinear_forward.  Arguments as in bitlinear_forward, with W_packed3 in
 * place of W_packed (16-byte aligned); no workspace.
 */
bitlinear_status bitlinear_forward_base3(const uint8_t* W_packed3, const float* gamma,
                                         int64_t N, int64_t K, const int8_t* X_q,
                                         const float* x_scale, const int32_t* x_sum,
                                         int64_t M, void* Y, bitlinear_dtype y_dtype,
                                         void* stream);

/*
 * Rewrites BLT3-v1 weights as BLT2-v1 (the same codes), e.g. for prefill with
 * bitlinear_forward.  W_packed3 as above (read only); W_packed
 * bitlinear_packed_bytes(N, K) bytes, device, 16-byte aligned (written).
 */
bitlinear_status bitlinear_base3_to_blt2(const uint8_t* W_packed3, int64_t N, int64_t K,
                                         uint8_t* W_packed, void* stream);

/* Kernels a forward call may launch (values of bitlinear_forward_kernel). */
typedef enum bitlinear_kernel {
  BITLINEAR_KERNEL_DECODE_DOT = 1, /* one token: dot products on the vector ALU */
  BITLINEAR_KERNEL_DECODE = 2,     /* up to 16 tokens: matrix instructions, weights streamed once */
  BITLINEAR_KERNEL_SKINNY = 3,     /* 2-64 tokens: activations and codes through an LDS ring
                                      (K split over workgroups on long-K shapes) */
  BITLINEAR_KERNEL_GEMM = 4,       /* tiled matrix product (K split over workgroups when tiles are few) */
  BITLINEAR_KERNEL_STREAM = 5,     /* one token, one persistent launch over every projection
                                      (bitlinear_forward_f32_multi; bitlinear_forward_f32 from
                                      2^25 weights) */
  BITLINEAR_KERNEL_FUSED_QUANT = 16 /* or'ed in: the activation quantiser runs in the same launch */
} bitlinear_kernel;

/*
 * Which kernel a forward call launches for these sizes, for profiling and
 * for callers that budget per kernel.  Host only: no GPU call, no state.
 * entry   0: bitlinear_forward / bitlinear_forward_grouped;
 *         1: bitlinear_forward_f32 / _f32_grouped;
 *         2: bitlinear_forward_rmsnorm / _rmsnorm_grouped.
 * M, K    as in those calls; G, N the group (G = 1, N = &n for one projection).
 * Returns a bitlinear_kernel value, with BITLINEAR_KERNEL_FUSED_QUANT or'ed
 * in when the quantiser (and normalisation) runs inside that launch; when it
 * is absent for entry 1 or 2 a quantiser launch comes first.  Returns
 * -BITLINEAR_ERR_SHAPE for sizes the call would reject (or an entry other
 * than 0, 1, 2).
 */
int bitlinear_forward_kernel(int entry, int64_t M, int G, const int64_t* N, int64_t K);

/*
 * How a bitlinear_forward_f32_multi call with these sizes runs (host only, no
 * GPU call): BITLINEAR_KERNEL_STREAM | BITLINEAR_KERNEL_FUSED_QUANT when all G
 * projections run as one launch (one token, every K[g] a multiple of 64 up to
 * 32768, and rows few enough per workgroup), 0 when they run one after
 * another (bitlinear_forward_kernel with entry 1 then names each projection's
 * kernel; with the shared quantiser launch, entry 0 does), -BITLINEAR_ERR_SHAPE
 * for sizes the call would reject.
 */
int bitlinear_forward_f32_multi_kernel(int64_t M, int G, const int64_t* N, const int64_t* K);

/* Static English name of a status. */
const char* bitlinear_status_string(bitlinear_status s);

/* Thread-local detail for the last non-OK status returned on this thread
 * ("" if none).  Valid until the next call on the same thread. */
const char* bitlinear_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
