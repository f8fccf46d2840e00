/*
 * rw4.h -- C ABI of the rotated W4A4 hot path on AMD Instinct MI355X (gfx950).
 *
 * The library computes, on one GPU, the online outlier-suppressing
 * activation transform followed by symmetric INT4 quantization in groups of
 * 128 channels, the matching offline weight transform + quantization, and
 * the W4A4 integer GEMM that consumes both:
 *
 *   Y[m, n] = sum over groups g of  sa[m, g] * sw[n, g] * acc[m, n, g],
 *   acc[m, n, g] = sum over k in g of  qa[m, k] * qw[n, k]   (exact int32).
 *
 * Sources (web pages, cited by title and section):
 *   - "Rotated Runtime Smooth: 训练无关的激活平滑器，用于精确的 INT4 推理"
 *     (isomlabs.com): problem definition (scale = max|X| / (2^(N-1)-1)),
 *     main equation (X_rot = X R, W_rot = R^-1 W, runtime smoothing scale
 *     s_j = max over tokens, Y = sum_j of partial products times s_j),
 *     term-by-term section (R = (1/sqrt(K)) [+-1], R R^T = I), Figure 4
 *     (group maximum = the GEMM block's smoothing scale, applied to the
 *     block's partial result), experimental setup (symmetric RTN).
 *   - "神经网络量化技术：Hadamard变换与格码本优化" (mhpn.cn), sections 2.1
 *     (Walsh-Hadamard matrix), 4.2 (butterfly factorization; H(AB) = (HA)B),
 *     6.1 (block Hadamard).
 *   - ParoQuant-style independent rotation article (codearts.csdn.net),
 *     sections 2.2 (layers of disjoint channel-pair rotations in each
 *     128-channel group), 2.3 (alpha = exp(beta) channel scale; 128-channel
 *     quantization groups), 3.2 (rotation patterns precompiled into a lookup
 *     table; rotate + scale + quantize fused in one kernel).
 *   - OstQuant page (rzmaituo.com), section 3.2: (X R D^-1)(D R^T W) = X W.
 *
 * Conventions used by every call:
 *   - Every pointer is a DEVICE pointer unless its name ends in _host.
 *   - Shapes: activations X [M, K] row-major with leading dimension ldx
 *     (elements); weights W given as [K, N] through element strides
 *     (stride_k, stride_n), so both [K, N] and [N, K] (nn.Linear) layouts
 *     work; output Y [M, N] row-major with leading dimension ldy.
 *     K must be a multiple of 128; G = K / 128 is the number of groups.
 *   - Packed INT4 (this library's layout; the pages fix none): codes lie in
 *     [-7, 7].  The INT4 range is [-8, 7] (Rotated Runtime Smooth page,
 *     problem definition), but the symmetric scale max/7 maps every value
 *     into [-7, 7] (-8 never arises), and this layout stores exactly that
 *     domain: a code of -8 cannot be represented.  Every 32-bit
 *     little-endian word w (bytes 4w..4w+3 of a row) carries the codes
 *     c_0..c_7 of channels 8w..8w+7 as sign-magnitude (|c| in 3 bits, sign
 *     1 = negative, zero with sign 0), and the words of each 16-byte chunk
 *     pair up as (4j, 4j+3) and (4j+1, 4j+2), sharing their bits: the
 *     pair's 16 codes (the first word's c_0..c_7 as k = 0..7, its
 *     partner's as k = 8..15) form the dense 96-bit string X of their FP6
 *     E2M3 encodings (code k, as the subnormal c/8, at bits 6k..6k+5:
 *     |c| in bits 0-2, sign in bit 5), and the pair's words a (first) and
 *     b (partner) hold
 *       a = (X[0:32] & A) | (X[32:64] & ~A),
 *       b = (X[64:96] & C) | (X[32:64] & ~C),  A = 0xE79E79E7, C = 0x9E79E79E,
 *     so X[0:32] = a & A, X[64:96] = b & C, X[32:64] = (a & ~A) | (b & ~C):
 *     the GEMM's operand form, opened with two masks.  Bit t of code k
 *     (t = 0, 1, 2 for |c|, 3 for the sign) sits in word (a or b) at bit:
 *       k  0-4: a:6k+(0,1,2,5);   k 5: a30 a31 b0 a3;  k 6: a4 b5 b6 a9;
 *       k 7: a10 b11 b12 a15;  k 8: a16 b17 b18 a21;  k 9: a22 b23 b24 a27;
 *       k 10: a28 b29 b30 b1;  k 11-15: b:6k-64+(0,1,2,5).
 *     qa is [M, K/2] bytes, qw is [N, K/2] bytes, rows contiguous.
 *   - Scales: fp32, row-major, sa [M, G], sw [N, G].
 *   - stream is a hipStream_t (NULL = the null stream).  Every call checks
 *     its arguments on the host, enqueues its kernels on `stream` and
 *     returns; the hot calls neither allocate nor synchronize.  A fault
 *     inside a kernel surfaces at the caller's next synchronization.
 *   - Ownership: the caller owns every tensor (inputs, outputs, the RRS
 *     workspace).  The library owns only a transform object (host struct +
 *     device lookup tables), allocated by rw4_transform_* and freed by
 *     rw4_transform_destroy.  Transforms are immutable after creation and
 *     may be shared across streams and threads.
 *   - Errors: no exceptions or aborts cross the ABI; every call returns a
 *     status.  M == 0 (or N == 0 for the GEMM and pack) is a valid no-op.
 *     Device pointers must be 16-byte aligned, and x's row pitch
 *     (ldx * element size) a multiple of 16 bytes.
 */
#ifndef RW4_H
#define RW4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RW4_OK = 0,
  RW4_ERR_ARG = 1,          /* null pointer, unknown enum, misaligned pointer/pitch, ld too small, bad pair table */
  RW4_ERR_SHAPE = 2,        /* K % 128 != 0, K != transform K, bad Hadamard block, layers < 1, negative size */
  RW4_ERR_UNSUPPORTED = 3,  /* valid but unimplemented combination (e.g. RRS with a Givens transform) */
  RW4_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed */
  RW4_ERR_NOMEM = 5         /* device allocation failed in rw4_transform_* */
} rw4_status;

typedef enum { RW4_F32 = 0, RW4_BF16 = 1 } rw4_dtype;

typedef enum {
  /* transform, then per-(token, 128-channel group) symmetric INT4:
     sa = max|x~| / 7 over the group, q = rne(x~ / sa).  |x~ / sa| <= 7, so
     the codes lie in [-7, 7], inside the INT4 range [-8, 7] (no clamp is
     needed; -8 never arises).  Rotated Runtime Smooth page, problem
     definition (scale = max|X| / (2^(N-1) - 1)) and experimental setup
     (symmetric round-to-nearest). */
  RW4_ACT_GROUP128 = 0,
  /* Rotated Runtime Smooth: transform, s_g = max over ALL M tokens and the
     group's channels of |x~|, z = x~ / s_g, per-token a_t = max_j |z| / 7,
     q = rne(z / a_t) in [-7, 7], stored scale sa[t, g] = a_t * s_g.
     Rotated Runtime Smooth page, main equation (runtime smoothing scale =
     channel maximum over the tokens) and Figure 4 (2) (the group maximum is
     the smoothing scale of the GEMM block). */
  RW4_ACT_RRS_PER_TOKEN = 1
} rw4_act_mode;

typedef struct rw4_transform rw4_transform; /* opaque */

/* Normalized block Walsh-Hadamard transform R = blockdiag(H_b / sqrt(b))
 * over K channels, H_b in Sylvester order ((H)_ij = (-1)^popcount(i AND j)).
 * Defined by: the QuIP#/QTIP page, section 2.1 (Walsh-Hadamard matrix from
 * the bit parity of the index pair), section 4.2 (butterfly factorization)
 * and section 6.1 (block Hadamard); the Rotated Runtime Smooth page,
 * term-by-term section (R = (1/sqrt(K)) [+-1], R R^T = I).
 * block: a power of two, 128 <= block <= K, block divides K.  Blocks larger
 * than 128 need K in {512, 1024, 2048, 4096, 8192} (else UNSUPPORTED).
 * Allocates nothing on the device.  *out receives the new transform. */
rw4_status rw4_transform_hadamard(int64_t K, int32_t block, void* stream, rw4_transform** out);

/* Randomized block Hadamard transform R = blockdiag(diag(d) H_b / sqrt(b)),
 * d a +-1 diagonal (the random sign diagonal the QuIP#/QTIP page pairs with
 * the Hadamard matrix; R stays orthogonal).  Activations x~ = x R (channel k
 * negated where d_k = -1, then the block transform); weights W~ = R^T W =
 * blockdiag(H_b / sqrt(b)) diag(d) W.
 *   signs_host [K] int8, every entry +1 or -1 (ARG otherwise); copied to a
 *   device table of K 32-bit words; the upload is synchronous with respect
 *   to `stream`.  block as for rw4_transform_hadamard. */
rw4_status rw4_transform_hadamard_signed(int64_t K, int32_t block, const int8_t* signs_host,
                                        void* stream, rw4_transform** out);

/* ParoQuant-style independent rotation (the ParoQuant-style article,
 * section 2.2: layers of disjoint channel-pair rotations in each group;
 * section 2.3: alpha = exp(beta); section 3.2: the rotation patterns kept in
 * a lookup table, only the angles supplied at run time): for each
 * 128-channel group g,
 * R_g = G_1 G_2 ... G_L, where layer l rotates up to 64 disjoint channel
 * pairs (i, j), i < j < 128, by angle theta: (xG)_i = c x_i + s x_j,
 * (xG)_j = -s x_i + c x_j; then channel scale alpha = exp(beta):
 * activations x~ = x R D^-1, weights W~ = D R^T W, D = diag(alpha).
 *   pairs_host [K/128][layers][64][2] uint8, 0xFF in both bytes = empty slot
 *   theta_host [K/128][layers][64] fp32 (ignored for empty slots)
 *   beta_host  [K] fp32 (exp(+-beta) must be finite and nonzero in fp32)
 * The host computes cos/sin/exp in double, rounds them to fp32, pads every
 * layer to a full matching with zero-angle pairs of the unused channels
 * (exactly the identity), and uploads the tables (176 KiB at K = 4096,
 * L = 8).  ARG if a pair is out of range, not i < j, or reuses a channel
 * inside its layer, or if an angle of a used slot or any beta is not
 * finite.  The upload is synchronous with respect to `stream`. */
rw4_status rw4_transform_givens(int64_t K, int32_t layers, const uint8_t* pairs_host,
                                const float* theta_host, const float* beta_host, void* stream,
                                rw4_transform** out);

/* The same transform with the angles stored in half precision (the
 * independent-rotation article keeps its trained angles in fp16): theta_f16
 * holds IEEE binary16 bit patterns, [K/128][layers][64]; every value is
 * widened exactly and must be finite (ARG otherwise).  Equivalent to
 * rw4_transform_givens with theta = the widened values. */
rw4_status rw4_transform_givens_f16(int64_t K, int32_t layers, const uint8_t* pairs_host,
                                    const uint16_t* theta_f16_host, const float* beta_host, void* stream,
                                    rw4_transform** out);

/* Transforms with device tables (signed Hadamard, Givens) accept K up to
 * 2^24 (RW4_ERR_SHAPE above) and must be used while the device that was
 * current at their creation is current (RW4_ERR_ARG otherwise); a host
 * allocation failure while building the tables is RW4_ERR_NOMEM. */

/* Frees the transform and its device tables.  The caller guarantees no
 * enqueued work still uses it.  NULL is a no-op. */
rw4_status rw4_transform_destroy(rw4_transform* t);

/* K of a transform (0 for NULL). */
int64_t rw4_transform_k(const rw4_transform* t);

/* quantize_act: one pass (two for RRS) over X [M, K] (x_dtype F32 or BF16,
 * leading dimension ldx elements): transform, quantize, pack.
 * Defined by: the Rotated Runtime Smooth page, main equation (X_rot = X R,
 * then runtime smoothing and quantization of the activations) and problem
 * definition (symmetric scale max|X| / 7 for INT4); the ParoQuant-style
 * article, section 3.2 (rotate, scale and quantize fused in one kernel) and
 * section 2.3 (groups of 128 channels share a scale; x R D^-1 with
 * D = diag(exp(beta))); the QuIP#/QTIP page, sections 2.1 (Walsh-Hadamard
 * matrix) and 6.1 (block Hadamard).
 * Input magnitude: the transform sums up to b inputs in fp32 before the
 * normalization (folded into the stored scale), so every block's sum of |x|
 * must stay below FLT_MAX: |x| <= 2.6e36 for b = 128 and <= 8.3e34 for
 * b = 4096 always suffices (bf16 inputs reach 3.4e38).  Larger inputs give
 * infinite scales; they are not detected.  Inputs must be finite: a NaN or
 * infinity spreads through the transform over its whole block, and the codes
 * and scales of the groups it reaches are unspecified (in RRS mode the group
 * maxima it reaches, and so every row's scales for those groups); no error is
 * reported.
 *   qa [M, K/2] uint8 packed codes (output)
 *   sa [M, K/128] fp32 scales (output)
 *   workspace: RRS only, >= K/128 fp32 device floats, 16-byte aligned,
 *     owned by the caller and overwritten (it receives s_g); NULL otherwise.
 * RRS needs a Hadamard transform (any block) with K in
 * {512, 1024, 2048, 4096, 8192}.  GROUP128 works with every transform. */
rw4_status rw4_quantize_act(const rw4_transform* t, rw4_act_mode mode, const void* x,
                            rw4_dtype x_dtype, int64_t M, int64_t ldx, uint8_t* qa, float* sa,
                            float* workspace, void* stream);

/* quantize_act_static: rw4_quantize_act with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops and harnesses that forbid allocation).  In RRS mode the
 * group maxima s_g live in a static array of the library, 64 floats per GPU
 * (so K <= 8192; RW4_ERR_SHAPE beyond), held by each GPU the library runs
 * on until the process ends; the call allocates nothing and clears what it
 * uses with a kernel.  Every call on one GPU shares that array, which keeps
 * the last call's contents: calls that overlap on one GPU (two streams, two
 * threads) race and must be serialized by the caller.  GROUP128 mode needs
 * no scratch and is exactly rw4_quantize_act.  Arguments, layouts and
 * errors otherwise as rw4_quantize_act. */
rw4_status rw4_quantize_act_static(const rw4_transform* t, rw4_act_mode mode, const void* x, rw4_dtype x_dtype,
                                   int64_t M, int64_t ldx, uint8_t* qa, float* sa, void* stream);

/* ---- Asymmetric (s, z) activation groups ---------------------------------
 * The independent-rotation article, section 2.3: a group of 128 channels
 * shares its quantization parameters (s, z); the Rotated Runtime Smooth
 * page's symbol table: q = round(x * scale) + offset.  Reading: min/max
 * round-to-nearest with zero kept inside the range.  Per (row, group g) of
 * the transformed row x~ (block-128 Hadamard only):
 *   lo = min(0, min x~), hi = max(0, max x~), s = (hi - lo) / 15,
 *   z = rne(-lo / s), q = clamp(rne(x~ / s) + z, 0, 15);  x~ ~ s (q - z).
 * qa [M][K/2]: unsigned codes in the paired form of rw4_quantize_act's
 * codes (NOT the same bits): the FP6 E2M3 encoding of u/8 is u itself
 * (bits 0-3), and the masks are A = 0xCF3CF3CF, C = 0x3CF3CF3C; bit t of
 * code k of a pair: k 0-4: a:6k+t;  k 5: a30 a31 b0 b1;  k 6-10:
 * a:6k-32+(0,1), b:6k-32+(2,3);  k 11-15: b:6k-64+t
 * (the same two-mask opening as the signed form); sa [M][K/128] fp32 scales s;
 * za [M][K/128] fp32 zero points (integers 0..15).  A group of zeros gets
 * s = 0, z = 0 and codes 0.  Arguments and errors otherwise as
 * rw4_quantize_act; other transforms: RW4_ERR_UNSUPPORTED. */
rw4_status rw4_quantize_act_asym(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M, int64_t ldx,
                                 uint8_t* qa, float* sa, float* za, void* stream);

/* cw [N][K/128] fp32 = the sum of the 128 codes of each group of the packed
 * weight rows qw [N][K/2] (rw4_pack_weight's form): what an asymmetric
 * activation's zero point multiplies.  Offline, with the weight pack.
 * K a multiple of 128, else RW4_ERR_SHAPE. */
rw4_status rw4_weight_code_sums(const uint8_t* qw, int64_t N, int64_t K, float* cw, void* stream);

/* y [M][N] = sum over g of sa[m,g] sw[n,g] sum over k in g of
 * (qa[m,k] - za[m,g]) qw[n,k], for the asymmetric activations above and
 * symmetric weights (groups of 128).  Computed as the integer products
 * minus za cw, exact, then the fp32 epilogue of rw4_w4a4_gemm; y fp32 or
 * bf16 (round to nearest even), ld ldy >= N.  Errors as rw4_w4a4_gemm. */
rw4_status rw4_w4a4_gemm_asym(const uint8_t* qa, const float* sa, const float* za, const uint8_t* qw,
                              const float* sw, const float* cw, int64_t M, int64_t N, int64_t K, void* y,
                              rw4_dtype y_dtype, int64_t ldy, void* stream);

/* out [M][K] = s (q - z) from the asymmetric form (the KV-cache read-back of
 * asymmetric groups), rounded once to fp32, then to bf16 when asked.
 * ldo >= K elements, 16-byte aligned rows.  Errors as rw4_dequantize. */
rw4_status rw4_dequantize_asym(const uint8_t* q, const float* s, const float* z, int64_t M, int64_t K, void* out,
                               rw4_dtype out_dtype, int64_t ldo, void* stream);

/* ---- 8-bit groups for extreme outliers ----------------------------------
 * The independent-rotation article, section 4.1: mixed precision, an 8-bit
 * representation kept for extreme outliers.  Reading: the caller names the
 * 128-channel groups (a per-layer choice, like the article's other
 * remedies for outlier-heavy layers).  Such a group is quantized
 * symmetrically with 225 levels, q8 = rne(112 x~ / max|x~|) in [-112, 112],
 * and split exactly as q8 = 15 h + l, h = rne(q8 / 15), h and l in [-7, 7]:
 * two INT4 planes that the INT4 GEMM multiplies by the same weights.
 *   slot_of_group [K/128] int32 (device): -1 for an INT4 group, j in
 *     [0, n8) for the j-th 8-bit group (values outside [-1, n8) act as -1);
 *   qa [M][(K + 128 n8)/2]: rw4_quantize_act's codes for INT4 groups; an
 *     8-bit group's h plane in its own place and its l plane as extra group
 *     K/128 + j;
 *   sa [M][K/128 + n8]: max/7 (scaled as rw4_quantize_act) for INT4 groups,
 *     15 max/112 for an h plane, max/112 for an l plane.
 * Block-128 Hadamard only (else RW4_ERR_UNSUPPORTED); n8 <= K/128. */
rw4_status rw4_quantize_act_mixed(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M, int64_t ldx,
                                  const int32_t* slot_of_group, int64_t n8, uint8_t* qa, float* sa, void* stream);

/* The matching weights: qw [N][K/2] and sw [N][K/128] (rw4_pack_weight)
 * copied to qw_ext [N][(K + 128 n8)/2] and sw_ext [N][K/128 + n8] with the
 * groups groups8[0..n8) (device int32, the 8-bit groups in slot order)
 * appended again; a listed group outside [0, K/128) gives zero codes and
 * scale.  Offline, with the weight pack.  rw4_w4a4_gemm over K + 128 n8 then
 * computes the layer. */
rw4_status rw4_extend_weight_groups(const uint8_t* qw, const float* sw, int64_t N, int64_t K, const int32_t* groups8,
                                    int64_t n8, uint8_t* qw_ext, float* sw_ext, void* stream);

/* ---- One decode step in one launch ---------------------------------------
 * y [M, N] = w4a4_gemm(quantize_act(t, x), qw, sw) for a decode-sized step
 * (1 <= M <= 16 tokens) in one kernel launch (the independent-rotation
 * article, section 3.2: rotate, scale and quantize in one kernel; the
 * QuIP#/QTIP page, section 6.1: precomputed fused kernels against launch
 * latency).  Each wave transforms and quantizes exactly the 128-channel
 * slices its own MFMAs consume; the codes never reach memory and nothing is
 * allocated.  Transform: the block-128 Hadamard, with or without random
 * signs (others: RW4_ERR_UNSUPPORTED; the Givens rotation, done in every
 * block, costs more than the launch it saves).  x as for rw4_quantize_act
 * (M <= 16, else RW4_ERR_SHAPE); qw/sw and y as for rw4_w4a4_gemm (group
 * 128).  The codes, scales and products are those of rw4_quantize_act and
 * rw4_w4a4_gemm, summed in the same order, so y equals those two calls in a
 * row. */
rw4_status rw4_decode_fused(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M, int64_t ldx,
                            const uint8_t* qw, const float* sw, int64_t N, void* y, rw4_dtype y_dtype, int64_t ldy,
                            void* stream);

/* ---- Rotated Runtime Smooth with the channel reorder --------------------
 * The Rotated Runtime Smooth page, Figure 4 (1): activations and weights are
 * reordered by the channel-wise maxima of the activations (Y is a sum over
 * channels, so the order does not change it); Figure 4 (2): the reordered
 * channels are grouped by the GEMM block and each group's maximum is its
 * runtime smoothing scale.  Readings: the maxima are taken over all M tokens
 * of the call; the order is by decreasing maximum, equal maxima by
 * increasing channel index; the weights are quantized per output channel
 * (the page's experimental setup), so reordering them only permutes codes.
 * One layer call:
 *   rw4_quantize_act_rrs_reorder(t, x, ..., qa, sa, order, ws)   activations
 *   rw4_permute_codes(qw, N, K, order, qw_ordered)               weights
 *   rw4_w4a4_gemm(qa, sa, qw_ordered, sw, ...)                   the product
 * with qw/sw from rw4_pack_weight_per_channel (offline). */

/* Bytes of device workspace rw4_quantize_act_rrs_reorder needs for K
 * channels (per-block channel maxima, the maxima, the group scales); 0 for
 * an invalid K. */
int64_t rw4_rrs_reorder_workspace_bytes(int64_t K);

/* Transform (a Hadamard transform, any block, plain or signed; K in {512,
 * 1024, 2048, 4096}, else RW4_ERR_UNSUPPORTED), per-channel maxima of
 * |x~| over the M tokens, channel order, smoothing by the reordered groups'
 * maxima, per-token INT4.  Writes qa [M, K/2] in the reordered channel
 * order, sa [M, K/128] (a_t * s_g of the reordered groups) and order [K]
 * int32 (order[r] = the channel placed at position r, a permutation).
 * workspace: rw4_rrs_reorder_workspace_bytes(K) bytes, 16-byte aligned,
 * owned by the caller, overwritten.  Other arguments as rw4_quantize_act. */
rw4_status rw4_quantize_act_rrs_reorder(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M,
                                        int64_t ldx, uint8_t* qa, float* sa, int32_t* order, void* workspace,
                                        void* stream);

/* pack_weight with one scale per output channel over all K (max / 7 of the
 * transformed row), stored in every one of the K/128 scale columns of sw.
 * Hadamard transforms with K in {512, ..., 8192} (else UNSUPPORTED).
 * Arguments as rw4_pack_weight. */
rw4_status rw4_pack_weight_per_channel(const rw4_transform* t, const void* w, rw4_dtype w_dtype, int64_t N,
                                       int64_t stride_k, int64_t stride_n, uint8_t* qw, float* sw, void* stream);

/* out[r, j] = code j' = order[j] of row r of q, for rows rows of K codes
 * (packed as everywhere, K % 128 == 0, K <= 8192); order is a permutation
 * of [0, K) (device int32 [K]; it is not checked: an index outside
 * [0, K) is clamped into it).  out must not alias q. */
rw4_status rw4_permute_codes(const uint8_t* q, int64_t rows, int64_t K, const int32_t* order, uint8_t* out,
                             void* stream);

/* pack_weight: W~ = R^T W (Hadamard) or D R^T W (Givens) for each of the N
 * output channels, then per-(channel, 128-group) symmetric INT4 and packing
 * (codes in [-7, 7], scale max / 7).  Defined by: the Rotated Runtime Smooth
 * page, main equation (W_rot = R^-1 W, R^-1 = R^T); the OstQuant page,
 * section 3.2 ((X R D^-1)(D R^T W) = X W); the QuIP#/QTIP page, section 4.2
 * (the transform folded into the weights offline, H(AB) = (HA)B); the
 * ParoQuant-style article, section 2.3 (W_hat = diag(alpha) W, 128-channel
 * groups).  The same input-magnitude bound as quantize_act applies.
 * Element (k, n) of W is w[k * stride_k + n * stride_n] (w_dtype F32/BF16;
 * strides in elements, > 0).
 *   qw [N, K/2] uint8 (output), sw [N, K/128] fp32 (output). */
rw4_status rw4_pack_weight(const rw4_transform* t, const void* w, rw4_dtype w_dtype, int64_t N,
                           int64_t stride_k, int64_t stride_n, uint8_t* qw, float* sw,
                           void* stream);

/* rotate_act: the transform alone, x~ = x R (Hadamard, plain or signed,
 * with the 1/sqrt(b) normalization) or x~ = x R D^-1 (Givens), written
 * unquantized as fp32 or bf16 (round to nearest even) into out [M, K]
 * (leading dimension ldo >= K elements, 16-byte aligned rows).  This is the
 * query side of an INT4 KV cache: keys are stored by quantize_act in the
 * rotated domain and read back by dequantize, queries are rotated by this
 * call, and (q R)(k R)^T = q k^T because R is orthogonal (the OstQuant page,
 * section 3.2: an extra Hadamard on queries and keys after RoPE; the
 * Rotated Runtime Smooth page, experimental setup: KV cache quantized in
 * groups of 128).  For Givens transforms (q R D^-1)(k R D^-1)^T differs
 * from q k^T by D^-2; such a transform is meant for weight products.
 *   x [M, K] (x_dtype F32 or BF16, ldx elements), same rules as
 *   quantize_act; any transform. */
rw4_status rw4_rotate_act(const rw4_transform* t, const void* x, rw4_dtype x_dtype, int64_t M, int64_t ldx,
                          void* out, rw4_dtype out_dtype, int64_t ldo, void* stream);

/* dequantize: x_hat[r, k] = code(q[r], k) * s[r, k / 128], the stored codes
 * times their group scale, in the transformed domain (for RRS the stored
 * scale already carries the smoothing factor); the complex-domain
 * quantization page, section 2.1: Q(x) = Delta * round(x / Delta).  Reads
 * back an INT4 KV cache written by quantize_act.  The product is rounded
 * to fp32, then (out_dtype BF16) to the nearest bf16, ties to even.
 *   q [M, K/2] packed codes, s [M, K/128] fp32 scales (as quantize_act
 *   writes them); out [M, K] row-major with leading dimension ldo >= K
 *   elements, 16-byte aligned rows.  K % 128 == 0. */
rw4_status rw4_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t K, void* out,
                          rw4_dtype out_dtype, int64_t ldo, void* stream);

/* w4a4_gemm: Y = sum over groups of sa * sw * (qa . qw^T restricted to the
 * group).  Defined by: the Rotated Runtime Smooth page, main equation (Y is
 * the sum of the per-channel partial products, each multiplied back by its
 * scale) and Figure 4 (3) (the GEMM block equals the quantization group and
 * the block's scale multiplies the block's partial result); the
 * ParoQuant-style article, section 2.3 (one scale per 128-channel group).
 * Each group's integer dot products are exact (FP6 matrix cores on the
 * codes as exact small values, fp32 accumulation of integers below 2^24); the per-group rescale and the sum over groups are fp32, the output
 * is rounded once to y_dtype (F32, or BF16 with round-to-nearest-even).
 * Any M >= 0, N >= 0; K % 128 == 0 and K <= 2^24 (RW4_ERR_SHAPE otherwise).
 *   y [M, N] with leading dimension ldy >= N elements (16-byte aligned
 *   pointer; rows whose byte stride is a multiple of 16 get wide stores). */
rw4_status rw4_w4a4_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                         int64_t M, int64_t N, int64_t K, void* y, rw4_dtype y_dtype,
                         int64_t ldy, void* stream);

/* ---- Group-size variants -------------------------------------------------
 * The same four calls with the quantization group as an argument (the
 * independent-rotation article, section 2.3, shares one set of quantization
 * parameters per group of 128 channels; 64 and 256 are the neighbouring
 * choices).  Scale arrays then hold K / group columns per row.  group must
 * be 64, 128 or 256 (RW4_ERR_ARG otherwise) and divide K (RW4_ERR_SHAPE);
 * group 128 is exactly the call without the suffix.  Supported beyond 128
 * (RW4_ERR_UNSUPPORTED otherwise):
 *   quantize_act_g  64 and 256 with a block-128 Hadamard transform (plain or
 *                   signed) in RW4_ACT_GROUP128 mode (per-group scales);
 *   pack_weight_g   64 and 256 with a block-128 Hadamard transform;
 *   w4a4_gemm_g     64 (each 64-wide K-half is rescaled on its own; the
 *                   large-product kernel then needs 96 KiB of LDS, one
 *                   block per CU) and 256 (the two 128-wide halves of a
 *                   group accumulate into one exact integer sum,
 *                   |sum| <= 256 * 49, before the rescale); K stays a
 *                   multiple of 128;
 *   dequantize_g    64 and 256.
 * The independent-rotation article gives outlier-heavy layers the smaller
 * group (64).  A 64-group INT4 KV cache is written with quantize_act_g and
 * read with dequantize_g. */
rw4_status rw4_quantize_act_g(const rw4_transform* t, rw4_act_mode mode, int32_t group, const void* x,
                              rw4_dtype x_dtype, int64_t M, int64_t ldx, uint8_t* qa, float* sa,
                              float* workspace, void* stream);
rw4_status rw4_pack_weight_g(const rw4_transform* t, int32_t group, const void* w, rw4_dtype w_dtype,
                             int64_t N, int64_t stride_k, int64_t stride_n, uint8_t* qw, float* sw,
                             void* stream);
rw4_status rw4_w4a4_gemm_g(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           int64_t M, int64_t N, int64_t K, int32_t group, void* y, rw4_dtype y_dtype,
                           int64_t ldy, void* stream);
rw4_status rw4_dequantize_g(const uint8_t* q, const float* s, int64_t M, int64_t K, int32_t group, void* out,
                            rw4_dtype out_dtype, int64_t ldo, void* stream);

/* Static description of a status code. */
const char* rw4_status_str(rw4_status s);

/* Library version, e.g. "0.1.0". */
const char* rw4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RW4_H */
