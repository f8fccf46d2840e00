"""Plain CPU oracle of the rotated W4A4 hot path (numpy, float64).

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code
with the HIP path: every transform here is an explicit dense matrix product
(no butterflies, no lookup tables, no fusion), every quantizer is the plain
formula, and the integer GEMM is a float64 matrix product of integer-valued
matrices (exact: every partial sum is an integer far below 2**53).

Sources (web pages; a reader has the pages, cited by title and section):
  [RRS]   "Rotated Runtime Smooth: 训练无关的激活平滑器，用于精确的 INT4 推理"
          (isomlabs.com analysis of the ICLR/OpenReview paper): problem
          definition (symmetric scale max|X|/(2^(N-1)-1)), main equation
          (rotate, runtime smooth, quantize, sum of s_j-scaled partial
          products), term-by-term section (R = (1/sqrt(K))[+-1], R R^T = I),
          Figure 4 (group max = block smoothing scale, scale applied to the
          block's partial result), experimental setup (symmetric RTN).
  [QuIP]  "神经网络量化技术：Hadamard变换与格码本优化" (mhpn.cn): section 2.1
          (Walsh-Hadamard matrix from the popcount of the index pair),
          section 4.2 (H(AB) = (HA)B, fold the transform into the weights),
          section 6.1 (block Hadamard).
  [Paro]  ParoQuant-style independent rotation article (codearts.csdn.net):
          section 2.2 (independent rotations: disjoint channel pairs inside
          each 128-channel group), section 2.3 (channel scale alpha =
          exp(beta), W_hat = diag(alpha) W; groups of 128 share quantization
          parameters), section 3.2 (rotate, scale, quantize in one pass).
  [OstQ]  "一种基于正交与缩放变换的大模型量化方法" (OstQuant, rzmaituo.com),
          section 3.2: (X R D^-1)(D R^T W) = X W.
  [Cplx]  complex-domain quantization article (zwxr.cn), section 2.1:
          Q(x) = Delta * round(x / Delta), Delta = max|x| / (2^(b-1) - 1).

Readings where the pages are silent or garbled (each is listed with its
reason in the design notes):
  * rounding is round-half-to-even (numpy ``rint``);
  * codes are clamped to [-7, 7] (the symmetric scale never leaves it);
  * an all-zero group gets scale 0 and codes 0 (no epsilon);
  * Hadamard in Sylvester order, (H)_ij = (-1)^popcount(i AND j), 1/sqrt(b)
    per side;
  * Givens layer: (xG)_i = c x_i + s x_j, (xG)_j = -s x_i + c x_j for i < j,
    layers applied first to last; activations x R D^-1, weights D R^T W;
  * Rotated Runtime Smooth: rotate first, then divide by the group maximum
    over all tokens of the call (group = 128 contiguous channels = the GEMM
    K-block), then per-token symmetric INT4; the stored activation scale of
    (token t, group g) is a_t * s_g;
  * the symmetric quantizer's codes lie in [-7, 7] (scale = max / 7), the
    range the packed form holds;
  * packed INT4 (the pages fix no layout): 4 bits per code, 8 codes per
    little-endian 32-bit word, each code as sign-magnitude (|c| in 3 bits,
    sign 1 for negative, zero with sign 0); the words of each 16-byte
    chunk pair up as (4j, 4j+3) and (4j+1, 4j+2), and a fixed table gives
    the positions of a pair's 16 codes' bits in its two words (the layout
    of the stored form, chosen so that a pair opens into 16 FP6 E2M3
    values with two masks);
  * 8-bit groups for extreme outliers ([Paro] section 4.1, mixed
    precision): the caller names the 128-channel groups; their codes are
    symmetric with 225 levels, q8 in [-112, 112] (scale max / 112), split
    exactly as q8 = 15 h + l with h, l in [-7, 7], two INT4 planes: h in
    place of the group (scale 15 s8), l in an extra group appended after
    the K channels (scale s8), against a weight matrix whose named groups
    are appended again;
  * asymmetric (s, z) groups ([Paro] section 2.3; the [RRS] symbol table's
    q = round(x * scale) + offset): min/max round-to-nearest with zero kept
    inside the range, unsigned codes 0..15 with an integer zero point,
    packed 4 bits per code by a second pair of position tables.

Shapes: X [M, K] (tokens x input channels), W [K, N], Y = X W [M, N];
group size g = 128, G = K / g.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 128
QMAX = 7      # 2^(4-1) - 1
QMIN = -QMAX  # symmetric: max / 7 never gives -8
UMAX = 15     # 2^4 - 1: asymmetric (affine) codes 0..15
Q8MAX = 112   # 8-bit groups: 15 * 7 + 7, the largest |q| that splits into two INT4 codes

__all__ = [
    "GROUP", "QMAX", "QMIN",
    "hadamard", "hadamard_block",
    "givens_layer", "givens_group_rotation",
    "act_transform_blocks", "weight_transform_blocks",
    "transform_act", "transform_weight",
    "quantize_groups", "quantize_rrs", "rrs_channel_order", "quantize_per_channel", "permute_codes",
    "quantize_groups_asym", "UMAX", "pack_uint4", "unpack_uint4", "dequantize_asym", "weight_code_sums",
    "w4a4_gemm_asym", "Q8MAX", "quantize_groups_mixed", "split_q8", "extend_weight_groups", "mixed_gemm_reference",
    "pack_int4", "unpack_int4", "SIGNED_PAIR_LAYOUT", "UNSIGNED_PAIR_LAYOUT", "CHUNK_PAIRS",
    "group_accumulators", "dequant_gemm",
    "round_bf16", "round_output", "dequantize", "round_dequant_output",
    "quantize_act", "pack_weight", "w4a4_gemm", "layer_forward",
]


# --------------------------------------------------------------------------
# Rotations
# --------------------------------------------------------------------------

def hadamard(n: int) -> np.ndarray:
    """Unnormalized Walsh-Hadamard matrix, entries (-1)^popcount(i AND j).

    [QuIP] section 2.1 builds H from the parity of the bit count of the
    index pair (the operator was lost in extraction; AND is the Sylvester
    ordering whose rows are the Walsh functions).  [RRS] term-by-term
    section: R = (1/sqrt(K)) [s_ij], s_ij in {-1, +1}.
    """
    if n < 1 or (n & (n - 1)):
        raise ValueError("Hadamard size must be a power of two")
    idx = np.arange(n, dtype=np.int64)
    bits = np.bitwise_count(np.bitwise_and.outer(idx, idx))
    return np.where(bits % 2 == 0, 1.0, -1.0)


def hadamard_block(b: int) -> np.ndarray:
    """Orthonormal block H_b / sqrt(b) ([RRS] R R^T = I; [QuIP] section 6.1 block form)."""
    return hadamard(b) / math.sqrt(b)


def givens_layer(g: int, pairs, thetas) -> np.ndarray:
    """Dense g x g matrix of one layer of disjoint pairwise rotations.

    [Paro] section 2.2: each layer rotates disjoint channel pairs of the
    group.  Convention (a reading): for pair (i, j), i < j, angle theta,
    G_ii = G_jj = cos(theta), G_ji = sin(theta), G_ij = -sin(theta), so the
    row vector x maps to (xG)_i = c x_i + s x_j, (xG)_j = -s x_i + c x_j.
    Slots whose index is 0xFF are empty.
    """
    G = np.eye(g)
    for (i, j), th in zip(pairs, thetas):
        i, j = int(i), int(j)
        if i == 0xFF or j == 0xFF:
            continue
        if not (0 <= i < j < g):
            raise ValueError(f"bad pair {(i, j)}")
        c, s = math.cos(float(th)), math.sin(float(th))
        G[i, i] = c
        G[j, j] = c
        G[j, i] = s
        G[i, j] = -s
    return G


def givens_group_rotation(pairs_g: np.ndarray, theta_g: np.ndarray, g: int = GROUP) -> np.ndarray:
    """R_gamma = G_1 G_2 ... G_L for one group (layers applied first to last)."""
    R = np.eye(g)
    for l in range(pairs_g.shape[0]):
        R = R @ givens_layer(g, pairs_g[l], theta_g[l])
    return R


def _rotation_blocks(spec: dict, K: int):
    """Yield (k0, k1, R_block, d) with d the per-channel scale alpha (ones for Hadamard).

    A Hadamard spec may carry "signs" (K values of +-1): the randomized
    Hadamard transform R = diag(signs) H_b / sqrt(b) per block, the random
    sign diagonal the QuIP#/QTIP page pairs with the Hadamard matrix
    (section 6.1 block form; a +-1 diagonal keeps R R^T = I).
    """
    kind = spec["kind"]
    if kind == "hadamard":
        b = int(spec["block"])
        if K % b:
            raise ValueError("block must divide K")
        R = hadamard_block(b)
        signs = spec.get("signs")
        if signs is not None:
            signs = np.asarray(signs, dtype=np.float64)
            if signs.shape != (K,) or not np.all(np.abs(signs) == 1.0):
                raise ValueError("signs must be K values of +1 or -1")
        for k0 in range(0, K, b):
            if signs is None:
                yield k0, k0 + b, R, np.ones(b)
            else:
                # randomized Hadamard: R = diag(signs) H_b / sqrt(b), still orthogonal
                yield k0, k0 + b, signs[k0:k0 + b, None] * R, np.ones(b)
    elif kind == "givens":
        pairs, theta, beta = spec["pairs"], spec["theta"], spec["beta"]
        for gi in range(K // GROUP):
            k0, k1 = gi * GROUP, (gi + 1) * GROUP
            R = givens_group_rotation(pairs[gi], theta[gi].astype(np.float64))
            yield k0, k1, R, np.exp(beta[k0:k1].astype(np.float64))
    else:
        raise ValueError(f"unknown transform {kind!r}")


def act_transform_blocks(spec: dict, K: int):
    """Yield (k0, k1, T) such that x_tilde[:, k0:k1] = X[:, k0:k1] @ T.

    Hadamard: T = H_b / sqrt(b).  Givens: T = R_gamma D_gamma^-1 with
    D = diag(alpha), alpha = exp(beta) ([Paro] section 2.3; activations take
    alpha^-1 after the rotation, [Paro] section 3.2 order: rotate, scale,
    quantize).
    """
    for k0, k1, R, d in _rotation_blocks(spec, K):
        yield k0, k1, R / d[None, :]


def weight_transform_blocks(spec: dict, K: int):
    """Yield (k0, k1, T_w) such that W_tilde[k0:k1, :] = T_w @ W[k0:k1, :].

    T_w = D R^T, the inverse of the activation block R D^-1 ([RRS] main
    equation W_rot = R^-1 W with R^-1 = R^T; [OstQ] section 3.2
    (X R D^-1)(D R^T W) = X W; [QuIP] section 4.2 folds the transform into
    the weights offline).
    """
    for k0, k1, R, d in _rotation_blocks(spec, K):
        yield k0, k1, d[:, None] * R.T


def transform_act(X: np.ndarray, spec: dict) -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    out = np.empty_like(X)
    for k0, k1, T in act_transform_blocks(spec, X.shape[1]):
        out[:, k0:k1] = X[:, k0:k1] @ T
    return out


def transform_weight(W: np.ndarray, spec: dict) -> np.ndarray:
    W = np.asarray(W, dtype=np.float64)
    out = np.empty_like(W)
    for k0, k1, T in weight_transform_blocks(spec, W.shape[0]):
        out[k0:k1, :] = T @ W[k0:k1, :]
    return out


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------

def _rtn(v: np.ndarray) -> np.ndarray:
    """Round half to even, clamp to the symmetric range [-7, 7] (a no-op for |v| <= 7)."""
    return np.clip(np.rint(v), QMIN, QMAX)


def quantize_groups(xt: np.ndarray, g: int = GROUP):
    """Per-(row, group) symmetric INT4: scale = max|x| / 7, q = clamp(rne(x / scale)).

    [RRS] problem definition: alpha = max(|X|) / (2^(N-1) - 1); [Cplx]
    section 2.1: Q(x) = Delta * round(x / Delta); [Paro] section 2.3: groups
    of 128 channels share their quantization parameters.  A group whose
    maximum is 0 gets scale 0 and codes 0.

    Returns (codes int8 [R, K], scales float64 [R, G], ratio float64 [R, K])
    where ``ratio`` = x / scale before rounding (0 where scale is 0), used
    by the tests to recognise rounding ties.
    """
    xt = np.asarray(xt, dtype=np.float64)
    R, K = xt.shape
    if K % g:
        raise ValueError("K must be a multiple of the group size")
    Gn = K // g
    xg = xt.reshape(R, Gn, g)
    scale = np.abs(xg).max(axis=2) / QMAX
    safe = np.where(scale > 0, scale, 1.0)
    ratio = np.where(scale[:, :, None] > 0, xg / safe[:, :, None], 0.0)
    codes = _rtn(ratio).astype(np.int8)
    return codes.reshape(R, K), scale, ratio.reshape(R, K)


def quantize_groups_asym(xt: np.ndarray, g: int = GROUP):
    """Per-(row, group) asymmetric (affine) INT4 with a shared (s, z) per group.

    [Paro] section 2.3: each group of 128 channels shares its quantization
    parameters (s, z); the [RRS] symbol table: q = round(x * scale) + offset,
    scale and offset fixed by the bit width and the value range.  Reading
    (min/max round-to-nearest, zero kept inside the range so that it is
    represented exactly):

      lo = min(0, min_k x_k),  hi = max(0, max_k x_k)
      s  = (hi - lo) / 15
      z  = rne(-lo / s)                      (an integer in [0, 15])
      q  = clamp(rne(x / s) + z, 0, 15)      x_hat = s (q - z)

    A group of zeros gets s = 0, z = 0 and codes 0.  Returns (codes uint8
    [R, K], s float64 [R, G], z int64 [R, G], ratio float64 [R, K] = x / s,
    zratio float64 [R, G] = -lo / s), the last two for recognising rounding
    ties in the tests.
    """
    xt = np.asarray(xt, dtype=np.float64)
    R, K = xt.shape
    if K % g:
        raise ValueError("K must be a multiple of the group size")
    Gn = K // g
    xg = xt.reshape(R, Gn, g)
    lo = np.minimum(xg.min(axis=2), 0.0)
    hi = np.maximum(xg.max(axis=2), 0.0)
    s = (hi - lo) / UMAX
    safe = np.where(s > 0, s, 1.0)
    zratio = np.where(s > 0, -lo / safe, 0.0)
    z = np.rint(zratio).astype(np.int64)
    ratio = np.where(s[:, :, None] > 0, xg / safe[:, :, None], 0.0)
    codes = np.clip(np.rint(ratio) + z[:, :, None], 0, UMAX)
    codes = np.where(s[:, :, None] > 0, codes, 0).astype(np.uint8)
    return codes.reshape(R, K), s, z, ratio.reshape(R, K), zratio


def split_q8(q8: np.ndarray):
    """q8 = 15 h + l with h, l in [-7, 7]: h = rne(q8 / 15) (q8 / 15 is never a tie,
    15 being odd), l = q8 - 15 h."""
    q8 = np.asarray(q8, dtype=np.int64)
    h = np.rint(q8 / 15.0).astype(np.int64)
    return h, q8 - 15 * h


def quantize_groups_mixed(xt: np.ndarray, groups8, g: int = GROUP):
    """Per-(row, group) symmetric INT4, with the groups named in ``groups8`` kept
    at 8 bits ([Paro] section 4.1: mixed precision, an 8-bit representation for
    extreme outliers).  Reading: an 8-bit group uses the symmetric scale
    s8 = max|x| / 112 and codes q8 = clamp(rne(x / s8), -112, 112) (225 levels,
    so that q8 splits exactly into two INT4 codes, see split_q8).

    Returns (q [R, K] int64: INT4 codes in 4-bit groups, q8 in 8-bit groups;
    scales [R, G]: max/7 or max/112; ratio x / scale [R, K])."""
    xt = np.asarray(xt, dtype=np.float64)
    R, K = xt.shape
    Gn = K // g
    codes, sc, ratio = quantize_groups(xt, g)
    codes = codes.astype(np.int64)
    for gi in groups8:
        sl = slice(gi * g, (gi + 1) * g)
        m = np.abs(xt[:, sl]).max(axis=1)
        s8 = m / Q8MAX
        safe = np.where(s8 > 0, s8, 1.0)
        r = np.where(s8[:, None] > 0, xt[:, sl] / safe[:, None], 0.0)
        codes[:, sl] = np.clip(np.rint(r), -Q8MAX, Q8MAX)
        sc[:, gi] = s8
        ratio[:, sl] = r
    return codes, sc, ratio


def extend_weight_groups(codes_w: np.ndarray, sw: np.ndarray, groups8, g: int = GROUP):
    """Weight codes [N, K] and scales [N, G] with the groups named in groups8
    appended again, in that order: [N, K + 128 n8], [N, G + n8]."""
    cw = np.asarray(codes_w)
    extra = [cw[:, gi * g:(gi + 1) * g] for gi in groups8]
    sw = np.asarray(sw)
    return (np.concatenate([cw] + extra, axis=1),
            np.concatenate([sw] + [sw[:, gi:gi + 1] for gi in groups8], axis=1))


def mixed_gemm_reference(q, sa, groups8, codes_w, sw, g: int = GROUP) -> np.ndarray:
    """Y = sum over groups of sa * sw * (sum of q * w) with q the mixed codes
    (INT4, or q8 in the 8-bit groups): the plain definition, float64."""
    return dequant_gemm(q, sa, codes_w, sw, g)


def dequantize_asym(codes: np.ndarray, s: np.ndarray, z: np.ndarray, g: int = GROUP) -> np.ndarray:
    """x_hat[r, k] = s[r, k // g] * (codes[r, k] - z[r, k // g]) (float64)."""
    c = np.asarray(codes, dtype=np.float64)
    return (c - np.repeat(np.asarray(z, dtype=np.float64), g, axis=1)) * np.repeat(
        np.asarray(s, dtype=np.float64), g, axis=1)


def quantize_rrs(xt: np.ndarray, g: int = GROUP, quantizer=None):
    """Rotated Runtime Smooth activation quantizer on already-rotated values.

    [RRS] main equation: s_j = max over tokens of |(X_rot)_j|, the smoothed
    activation X_rot diag(s)^-1 is quantized, and each channel's partial
    product is multiplied back by s_j.  [RRS] Figure 4 (2): channels are
    grouped by the GEMM block and the group's maximum is the group's
    smoothing scale.  [RRS] experimental setup: activations use symmetric
    RTN, here per token over the whole smoothed row.

      s_g    = max over all tokens t and channels j in g of |xt[t, j]|
      z      = xt / s_g(j)                (0 where s_g = 0)
      a_t    = max_j |z[t, j]| / 7
      q      = clamp(rne(z / a_t), -7, 7) (0 where a_t = 0)
      sa[t, g] = a_t * s_g

    ``quantizer`` replaces the INT4 rounding when given (a test hook: the
    identity turns the whole path into X W).  Returns (codes, sa, s, ratio).
    """
    xt = np.asarray(xt, dtype=np.float64)
    R, K = xt.shape
    Gn = K // g
    s = np.abs(xt.reshape(R, Gn, g)).max(axis=(0, 2))
    s_ch = np.repeat(s, g)
    z = np.where(s_ch[None, :] > 0, xt / np.where(s_ch > 0, s_ch, 1.0)[None, :], 0.0)
    a = np.abs(z).max(axis=1) / QMAX
    ratio = np.where(a[:, None] > 0, z / np.where(a > 0, a, 1.0)[:, None], 0.0)
    if quantizer is None:
        codes = _rtn(ratio).astype(np.int8)
    else:
        codes = quantizer(ratio)
    sa = a[:, None] * s[None, :]
    return codes, sa, s, ratio


def rrs_channel_order(xt: np.ndarray):
    """Channel order of the Rotated Runtime Smooth reorder.

    [RRS] Figure 4 (1): activations and weights are reordered by the
    channel-wise maxima of the activations (the reorder leaves Y unchanged,
    Y being a sum over channels in any order); Figure 4 (2): the reordered
    channels are then grouped by the GEMM block.  Reading: the maxima are
    taken over all tokens of the call, m_j = max_t |xt[t, j]|, and channels
    are sorted by decreasing m_j, equal maxima in increasing channel index
    (a stable sort), so channels of similar magnitude share a group.
    Returns (order, m): order[r] = the channel placed at position r.
    """
    xt = np.asarray(xt, dtype=np.float64)
    m = np.abs(xt).max(axis=0)
    order = np.argsort(-m, kind="stable")
    return order, m


def quantize_per_channel(wt_rows: np.ndarray):
    """Per-row symmetric INT4 over the whole row: scale = max|row| / 7 (the
    per-channel weight scheme of the [RRS] experimental setup, one scale per
    output channel).  Returns (codes, scale [R], ratio)."""
    x = np.asarray(wt_rows, dtype=np.float64)
    scale = np.abs(x).max(axis=1) / QMAX
    safe = np.where(scale > 0, scale, 1.0)
    ratio = np.where(scale[:, None] > 0, x / safe[:, None], 0.0)
    return _rtn(ratio).astype(np.int8), scale, ratio


# --------------------------------------------------------------------------
# Packing
# --------------------------------------------------------------------------

# The stored form: 4 bits per code, 8 codes per little-endian 32-bit word
# (code e of word w = channel 8 w + e of the row), the words of each 16-byte
# chunk paired as (4 j, 4 j + 3) and (4 j + 1, 4 j + 2).  A pair holds the
# 16 codes of its two words (k = 0..7 those of the first word, the one whose
# index has bit 1 clear, 8..15 those of its partner); the table below gives,
# for bit t of code k ((|c| bit 0, bit 1, bit 2, sign) signed, bits 0-3
# unsigned), the word of the pair (0 first, 1 partner) and the bit position
# in it.  No page fixes a layout.  This one is built so that, with f_k the
# 6-bit FP6 E2M3 encoding of code k (sign, two zero exponent bits, the
# magnitude as subnormal mantissa: the value c / 8; an unsigned u <= 15 is
# the E2M3 encoding of u / 8 with a zero sign bit), the dense 96-bit string
# sum_k f_k << 6 k splits into its three 32-bit words as
#   D0 = a & A,  D2 = b & C,  D1 = (a & ~A) | (b & ~C)
# for the pair's words a, b, with masks A = 0xE79E79E7, C = 0x9E79E79E
# (signed) and A = 0xCF3CF3CF, C = 0x3CF3CF3C (unsigned).  The tests pin the
# tables to this identity by brute force.
SIGNED_PAIR_LAYOUT = (
    ((0, 0), (0, 1), (0, 2), (0, 5)), ((0, 6), (0, 7), (0, 8), (0, 11)),
    ((0, 12), (0, 13), (0, 14), (0, 17)), ((0, 18), (0, 19), (0, 20), (0, 23)),
    ((0, 24), (0, 25), (0, 26), (0, 29)), ((0, 30), (0, 31), (1, 0), (0, 3)),
    ((0, 4), (1, 5), (1, 6), (0, 9)), ((0, 10), (1, 11), (1, 12), (0, 15)),
    ((0, 16), (1, 17), (1, 18), (0, 21)), ((0, 22), (1, 23), (1, 24), (0, 27)),
    ((0, 28), (1, 29), (1, 30), (1, 1)), ((1, 2), (1, 3), (1, 4), (1, 7)),
    ((1, 8), (1, 9), (1, 10), (1, 13)), ((1, 14), (1, 15), (1, 16), (1, 19)),
    ((1, 20), (1, 21), (1, 22), (1, 25)), ((1, 26), (1, 27), (1, 28), (1, 31)),
)
UNSIGNED_PAIR_LAYOUT = (
    ((0, 0), (0, 1), (0, 2), (0, 3)), ((0, 6), (0, 7), (0, 8), (0, 9)),
    ((0, 12), (0, 13), (0, 14), (0, 15)), ((0, 18), (0, 19), (0, 20), (0, 21)),
    ((0, 24), (0, 25), (0, 26), (0, 27)), ((0, 30), (0, 31), (1, 0), (1, 1)),
    ((0, 4), (0, 5), (1, 6), (1, 7)), ((0, 10), (0, 11), (1, 12), (1, 13)),
    ((0, 16), (0, 17), (1, 18), (1, 19)), ((0, 22), (0, 23), (1, 24), (1, 25)),
    ((0, 28), (0, 29), (1, 30), (1, 31)), ((1, 2), (1, 3), (1, 4), (1, 5)),
    ((1, 8), (1, 9), (1, 10), (1, 11)), ((1, 14), (1, 15), (1, 16), (1, 17)),
    ((1, 20), (1, 21), (1, 22), (1, 23)), ((1, 26), (1, 27), (1, 28), (1, 29)),
)
# word pairs of a 16-byte chunk (first word, partner)
CHUNK_PAIRS = ((0, 3), (1, 2))


def _pack_words(bits: np.ndarray, layout) -> np.ndarray:
    """bits [..., K, 4] (0/1) -> bytes [..., K/2] through the pair table."""
    if bits.shape[-2] % 32:
        raise ValueError("row length must be a multiple of 32 codes (16-byte chunks)")
    nc = bits.shape[-2] // 32
    b = bits.reshape(bits.shape[:-2] + (nc, 4, 8, 4)).astype(np.uint64)
    words = np.zeros(bits.shape[:-2] + (nc, 4), dtype=np.uint64)
    for first, partner in CHUNK_PAIRS:
        own = (first, partner)
        for k in range(16):
            src = own[k // 8]
            for t in range(4):
                role, pos = layout[k][t]
                words[..., own[role]] |= b[..., src, k % 8, t] << np.uint64(pos)
    out = np.empty(words.shape + (4,), dtype=np.uint8)
    for k in range(4):
        out[..., k] = (words >> np.uint64(8 * k)) & np.uint64(0xFF)
    return out.reshape(bits.shape[:-2] + (nc * 16,))


def _unpack_words(packed: np.ndarray, layout) -> np.ndarray:
    """bytes [..., 16 C] -> bits [..., 32 C, 4] through the pair table."""
    p = np.asarray(packed, dtype=np.uint8)
    if p.shape[-1] % 16:
        raise ValueError("packed row length must be a multiple of 16 bytes")
    nc = p.shape[-1] // 16
    q = p.reshape(p.shape[:-1] + (nc, 4, 4)).astype(np.uint64)
    words = q[..., 0] | (q[..., 1] << np.uint64(8)) | (q[..., 2] << np.uint64(16)) | (q[..., 3] << np.uint64(24))
    bits = np.zeros(p.shape[:-1] + (nc, 4, 8, 4), dtype=np.int64)
    for first, partner in CHUNK_PAIRS:
        own = (first, partner)
        for k in range(16):
            dst = own[k // 8]
            for t in range(4):
                role, pos = layout[k][t]
                bits[..., dst, k % 8, t] = ((words[..., own[role]] >> np.uint64(pos)) & np.uint64(1)).astype(np.int64)
    return bits.reshape(p.shape[:-1] + (nc * 32, 4))


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """[R, K] codes in [-7, 7] -> [R, K/2] bytes, K a multiple of 32.

    Sign-magnitude, 4 bits per code, 8 codes c_0..c_7 per little-endian
    32-bit word (bytes 4w..4w+3 of the row); the bits of the codes of a word
    pair (|c| bit 0, 1, 2 and the sign, 1 = negative) sit where
    SIGNED_PAIR_LAYOUT puts them.  Zero is always stored with sign 0.
    """
    c = np.asarray(codes)
    if c.min(initial=0) < QMIN or c.max(initial=0) > QMAX:
        raise ValueError("code out of the symmetric INT4 range [-7, 7]")
    c = c.astype(np.int64)
    mag = np.abs(c)
    bits = np.stack([mag & 1, (mag >> 1) & 1, (mag >> 2) & 1, (c < 0).astype(np.int64)], axis=-1)
    return _pack_words(bits, SIGNED_PAIR_LAYOUT)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: int8 codes [R, 2 * bytes]."""
    bits = _unpack_words(packed, SIGNED_PAIR_LAYOUT)
    mag = bits[..., 0] | (bits[..., 1] << 1) | (bits[..., 2] << 2)
    return np.where(bits[..., 3] == 1, -mag, mag).astype(np.int8)


def pack_uint4(codes: np.ndarray) -> np.ndarray:
    """[R, K] unsigned codes 0..15 -> [R, K/2] bytes (the asymmetric form), K a
    multiple of 32: 8 codes per little-endian 32-bit word, the bits of a word
    pair's codes where UNSIGNED_PAIR_LAYOUT puts them."""
    c = np.asarray(codes)
    if c.min(initial=0) < 0 or c.max(initial=0) > UMAX:
        raise ValueError("code out of the unsigned INT4 range [0, 15]")
    c = c.astype(np.int64)
    bits = np.stack([(c >> t) & 1 for t in range(4)], axis=-1)
    return _pack_words(bits, UNSIGNED_PAIR_LAYOUT)


def unpack_uint4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_uint4: uint8 codes [R, 2 * bytes]."""
    bits = _unpack_words(packed, UNSIGNED_PAIR_LAYOUT)
    return (bits[..., 0] | (bits[..., 1] << 1) | (bits[..., 2] << 2) | (bits[..., 3] << 3)).astype(np.uint8)


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------

def group_accumulators(qa: np.ndarray, qw: np.ndarray, g: int = GROUP) -> np.ndarray:
    """acc[m, n, gamma] = sum over k in group gamma of qa[m, k] * qw[n, k].

    qa [M, K] and qw [N, K] are unpacked integer codes.  float64 products of
    integer-valued matrices are exact here (|partial sums| <= K * 64 << 2^53).
    Returns int64 [M, N, G]; meant for small shapes.
    """
    qa = np.asarray(qa, dtype=np.float64)
    qw = np.asarray(qw, dtype=np.float64)
    M, K = qa.shape
    Gn = K // g
    acc = np.empty((M, qw.shape[0], Gn), dtype=np.int64)
    for gi in range(Gn):
        sl = slice(gi * g, (gi + 1) * g)
        acc[:, :, gi] = (qa[:, sl] @ qw[:, sl].T).astype(np.int64)
    return acc


def dequant_gemm(qa: np.ndarray, sa: np.ndarray, qw: np.ndarray, sw: np.ndarray,
                 g: int = GROUP) -> np.ndarray:
    """Y[m, n] = sum over gamma of sa[m, gamma] * sw[n, gamma] * acc[m, n, gamma] (float64).

    [RRS] main equation: the sum of per-channel partial products, each
    multiplied back by its scale; [RRS] Figure 4 (3): the block size equals
    the group size and the scale multiplies the block's partial result.
    """
    qa = np.asarray(qa, dtype=np.float64)
    qw = np.asarray(qw, dtype=np.float64)
    sa = np.asarray(sa, dtype=np.float64)
    sw = np.asarray(sw, dtype=np.float64)
    M, K = qa.shape
    Y = np.zeros((M, qw.shape[0]))
    for gi in range(K // g):
        sl = slice(gi * g, (gi + 1) * g)
        acc = qa[:, sl] @ qw[:, sl].T
        Y += (sa[:, gi][:, None] * sw[:, gi][None, :]) * acc
    return Y


def weight_code_sums(qw_packed, g: int = GROUP) -> np.ndarray:
    """cw[n, gamma] = sum over k in group gamma of the weight codes (int64), the
    per-group totals an asymmetric activation's zero point multiplies."""
    c = unpack_int4(qw_packed).astype(np.int64)
    N, K = c.shape
    return c.reshape(N, K // g, g).sum(axis=2)


def w4a4_gemm_asym(qa_packed, sa, za, qw_packed, sw, out_dtype: str = "f32") -> np.ndarray:
    """Oracle of the GEMM with asymmetric activations: the activation codes are
    centred by their group's zero point, then the symmetric GEMM's definition:
    Y[m, n] = sum over gamma of sa[m, gamma] * sw[n, gamma] * sum over k in gamma
    of (qa[m, k] - za[m, gamma]) * qw[n, k], in exact integers and float64."""
    qa = unpack_uint4(qa_packed).astype(np.int64)
    g = qa.shape[1] // np.asarray(sa).shape[1]
    centred = qa - np.repeat(np.asarray(za, dtype=np.int64), g, axis=1)
    Y = dequant_gemm(centred, sa, unpack_int4(qw_packed), sw, g)
    return round_output(Y, out_dtype)


def round_bf16(y: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bfloat16 value (ties to even), as float64.

    bfloat16 is the binary format with 8 exponent bits (as fp32) and 7
    fraction bits: 8 significant bits for normal values, and below 2^-126
    the subnormal grid with spacing 2^-133.  Inputs must lie below the bf16
    maximum."""
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)  # y = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(y, -q)), q)


def round_output(y: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return y.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(y)
    if dtype == "f64":
        return y
    raise ValueError(dtype)


def dequantize(codes: np.ndarray, scales: np.ndarray, g: int = GROUP) -> np.ndarray:
    """x_hat[r, k] = codes[r, k] * scales[r, k // g] (float64), the inverse of
    the quantizer up to rounding: Q(x) = Delta * round(x / Delta) ([Cplx]
    section 2.1), in the transformed domain (for RRS the stored scale a_t * s_g
    already carries the smoothing factor)."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    return c * np.repeat(s, g, axis=1)


def round_dequant_output(x: np.ndarray, dtype: str) -> np.ndarray:
    """Output rounding of the library's dequantize: the code * scale product is
    rounded to fp32 (it needs up to 27 significant bits), then, for bf16,
    rounded again to the nearest bf16 (ties to even)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return round_bf16(x32)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# The three library calls, as plain definitions
# --------------------------------------------------------------------------

def quantize_act(X: np.ndarray, spec: dict, mode: str = "group128", g: int = GROUP, order=None):
    """Oracle of quantize_act: transform, then per-group or RRS per-token INT4.

    ``g`` is the quantization group ([Paro] section 2.3 uses 128; other
    group sizes are a knob of the same quantizer).  Mode "group128_asym" is
    the asymmetric (s, z) quantizer (quantize_groups_asym; the dict also
    holds za and zratio, qa holds plain unsigned nibbles).  Mode
    "group128_mixed" keeps the groups listed in ``order`` at 8 bits
    (quantize_groups_mixed): qa [M, (K + 128 n8) / 2] holds the INT4 codes
    with each 8-bit group's h plane in place and its l planes appended, sa
    [M, G + n8] their scales; codes/scales hold the unsplit codes.  Mode "rrs_reorder" is
    Rotated Runtime Smooth with the channel reorder of [RRS] Figure 4 (1):
    the transformed channels are permuted by ``order`` (default: the
    rrs_channel_order of this call's activations) before grouping, and the
    codes are stored in that order.  Returns dict(qa=packed uint8 [M, K/2],
    sa=float64 [M, K/g], codes, ratio, xt=transformed activations, s=RRS
    group scales or None, order=the channel order or None, m=channel maxima
    or None).
    """
    xt = transform_act(X, spec)
    m = None
    if mode == "group128_mixed":
        # 8-bit groups as two INT4 planes: h in place, l appended (scales 15 s8 and s8)
        groups8 = list(order if order is not None else [])
        q, sc, ratio = quantize_groups_mixed(xt, groups8, g)
        planes = q.copy()
        sa_ext = [sc.copy()]
        lows = []
        for gi in groups8:
            sl = slice(gi * g, (gi + 1) * g)
            h, lo = split_q8(q[:, sl])
            planes[:, sl] = h
            sa_ext[0][:, gi] = 15.0 * sc[:, gi]
            lows.append(lo)
            sa_ext.append(sc[:, gi:gi + 1])
        ext = np.concatenate([planes] + lows, axis=1).astype(np.int8)
        return {"qa": pack_int4(ext), "sa": np.concatenate(sa_ext, axis=1), "codes": q, "scales": sc,
                "ratio": ratio, "xt": xt, "s": None, "order": groups8, "m": None}
    if mode == "group128_asym":
        codes, sa, za, ratio, zratio = quantize_groups_asym(xt, g)
        return {"qa": pack_uint4(codes), "sa": sa, "za": za, "codes": codes, "ratio": ratio, "zratio": zratio,
                "xt": xt, "s": None, "order": None, "m": None}
    if mode == "group128":
        codes, sa, ratio = quantize_groups(xt, g)
        s = None
    elif mode == "rrs":
        codes, sa, s, ratio = quantize_rrs(xt, g)
    elif mode == "rrs_reorder":
        if order is None:
            order, m = rrs_channel_order(xt)
        order = np.asarray(order)
        codes, sa, s, ratio = quantize_rrs(xt[:, order], g)
    else:
        raise ValueError(mode)
    return {"qa": pack_int4(codes), "sa": sa, "codes": codes, "ratio": ratio, "xt": xt, "s": s,
            "order": order if mode == "rrs_reorder" else None, "m": m}


def pack_weight(W: np.ndarray, spec: dict, g: int = GROUP, per_channel: bool = False):
    """Oracle of pack_weight: W_tilde = T_w W, per-(output channel, group) INT4.

    W is [K, N].  Returns dict(qw=packed uint8 [N, K/2], sw=float64 [N, K/g],
    codes [N, K], ratio [N, K], wt=W_tilde [K, N]).  ``per_channel`` uses one
    scale per output channel over all K ([RRS] experimental setup: weights
    per-channel symmetric), stored repeated in every group column, so that
    a permutation of the K channels only permutes the codes.
    """
    wt = transform_weight(W, spec)
    if per_channel:
        codes, scale, ratio = quantize_per_channel(wt.T)
        sw = np.repeat(scale[:, None], wt.shape[0] // g, axis=1)
    else:
        codes, sw, ratio = quantize_groups(wt.T, g)
    return {"qw": pack_int4(codes), "sw": sw, "codes": codes, "ratio": ratio, "wt": wt}


def permute_codes(codes: np.ndarray, order) -> np.ndarray:
    """Codes of every row taken in channel order ``order``: out[r, j] = codes[r, order[j]]
    (the weight side of the [RRS] Figure 4 (1) reorder)."""
    return np.asarray(codes)[:, np.asarray(order)]


def w4a4_gemm(qa_packed, sa, qw_packed, sw, out_dtype: str = "f32") -> np.ndarray:
    """Oracle of w4a4_gemm: unpack, exact grouped integer products, float64 epilogue, output rounding.

    The group size is K divided by the number of scale columns."""
    qa = unpack_int4(qa_packed)
    g = qa.shape[1] // np.asarray(sa).shape[1]
    Y = dequant_gemm(qa, sa, unpack_int4(qw_packed), sw, g)
    return round_output(Y, out_dtype)


def layer_forward(X, W, spec, mode="group128", out_dtype="f64"):
    """Whole layer: quantize_act, pack_weight, w4a4_gemm."""
    a = quantize_act(X, spec, mode)
    w = pack_weight(W, spec)
    return w4a4_gemm(a["qa"], a["sa"], w["qw"], w["sw"], out_dtype), a, w
