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
 *     [-7, 7] (the symmetric scale max/7 never leaves it).  Every 32-bit
 *     little-endian word (bytes 4w..4w+3 of a row) holds codes c_0..c_7 of
 *     that word as sign-magnitude nibbles: nibble e (byte e/2, low nibble
 *     for even e) = |c_e| in bits 0-2 plus the sign (1 = negative) of
 *     c_((e-1) mod 8) in bit 3; zero has sign 0.  Masking a word with
 *     0x87878787, and its rotation right by 4 bits likewise, gives the even
 *     and the odd codes as sign-magnitude bytes.
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
     sa = max|x~| / 7 over the group, q = clamp(rne(x~ / sa), -8, 7) */
  RW4_ACT_GROUP128 = 0,
  /* Rotated Runtime Smooth: transform, s_g = max over ALL M tokens and the
     group's channels of |x~|, z = x~ / s_g, per-token a_t = max_j |z| / 7,
     q = clamp(rne(z / a_t), -8, 7), stored scale sa[t, g] = a_t * s_g */
  RW4_ACT_RRS_PER_TOKEN = 1
} rw4_act_mode;

typedef struct rw4_transform rw4_transform; /* opaque */

/* Normalized block Walsh-Hadamard transform R = blockdiag(H_b / sqrt(b))
 * over K channels, H_b in Sylvester order ((H)_ij = (-1)^popcount(i AND j)).
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

/* ParoQuant-style independent rotation: for each 128-channel group g,
 * R_g = G_1 G_2 ... G_L, where layer l rotates up to 64 disjoint channel
 * pairs (i, j), i < j < 128, by angle theta: (xG)_i = c x_i + s x_j,
 * (xG)_j = -s x_i + c x_j; then channel scale alpha = exp(beta):
 * activations x~ = x R D^-1, weights W~ = D R^T W, D = diag(alpha).
 *   pairs_host [K/128][layers][64][2] uint8, 0xFF in both bytes = empty slot
 *   theta_host [K/128][layers][64] fp32 (ignored for empty slots)
 *   beta_host  [K] fp32
 * The host computes cos/sin/exp in double, rounds them to fp32, pads every
 * layer to a full matching with zero-angle pairs of the unused channels
 * (exactly the identity), and uploads the tables (176 KiB at K = 4096,
 * L = 8).  ARG if a pair is out of range, not i < j, or reuses a channel
 * inside its layer.  The upload is synchronous with respect to `stream`. */
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
 *   qa [M, K/2] uint8 packed codes (output)
 *   sa [M, K/128] fp32 scales (output)
 *   workspace: RRS only, >= K/128 fp32 device floats, 16-byte aligned,
 *     owned by the caller and overwritten (it receives s_g); NULL otherwise.
 * RRS needs a Hadamard transform (any block) with K in
 * {512, 1024, 2048, 4096, 8192}.  GROUP128 works with every transform. */
rw4_status rw4_quantize_act(const rw4_transform* t, rw4_act_mode mode, const void* x,
                            rw4_dtype x_dtype, int64_t M, int64_t ldx, uint8_t* qa, float* sa,
                            float* workspace, void* stream);

/* pack_weight: W~ = R^T W (Hadamard) or D R^T W (Givens) for each of the N
 * output channels, then per-(channel, 128-group) symmetric INT4 and packing.
 * Element (k, n) of W is w[k * stride_k + n * stride_n] (w_dtype F32/BF16;
 * strides in elements, > 0).
 *   qw [N, K/2] uint8 (output), sw [N, K/128] fp32 (output). */
rw4_status rw4_pack_weight(const rw4_transform* t, const void* w, rw4_dtype w_dtype, int64_t N,
                           int64_t stride_k, int64_t stride_n, uint8_t* qw, float* sw,
                           void* stream);

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
 * group).  Each group's integer dot products are exact (FP8 matrix cores on
 * the codes as exact small values, fp32 accumulation of integers below
 * 2^24); the per-group rescale and the sum over groups are fp32, the output
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
