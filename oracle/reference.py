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
  * packed INT4 (the pages fix no layout): sign-magnitude nibbles, 8 codes
    per little-endian 32-bit word; nibble e (byte e // 2, low nibble for
    even e) holds |c_e| in bits 0-2 and the sign of c_((e-1) mod 8) in bit 3.

Shapes: X [M, K] (tokens x input channels), W [K, N], Y = X W [M, N];
group size g = 128, G = K / g.
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 128
QMAX = 7      # 2^(4-1) - 1
QMIN = -QMAX  # symmetric: max / 7 never gives -8

__all__ = [
    "GROUP", "QMAX", "QMIN",
    "hadamard", "hadamard_block",
    "givens_layer", "givens_group_rotation",
    "act_transform_blocks", "weight_transform_blocks",
    "transform_act", "transform_weight",
    "quantize_groups", "quantize_rrs",
    "pack_int4", "unpack_int4",
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


# --------------------------------------------------------------------------
# Packing
# --------------------------------------------------------------------------

def pack_int4(codes: np.ndarray) -> np.ndarray:
    """[R, K] codes in [-7, 7] -> [R, K/2] bytes, K a multiple of 8.

    Sign-magnitude nibbles, 8 codes c_0..c_7 per little-endian 32-bit word
    (bytes 4w..4w+3 of the row): nibble e of the word (byte e // 2, low
    nibble for even e) holds |c_e| in its bits 0-2, and its bit 3 holds the
    sign (1 = negative) of the code before it, c_((e-1) mod 8).  Zero is
    always stored with sign 0.  (No page fixes a packed layout; this one
    lets a reader split a word into two 4-byte groups of sign-magnitude
    bytes with one mask and one rotate + mask.)
    """
    c = np.asarray(codes)
    if c.shape[-1] % 8:
        raise ValueError("row length must be a multiple of 8")
    if c.min(initial=0) < QMIN or c.max(initial=0) > QMAX:
        raise ValueError("code out of the symmetric INT4 range [-7, 7]")
    c = c.astype(np.int64)
    words = c.reshape(c.shape[:-1] + (c.shape[-1] // 8, 8))
    mag = np.abs(words)
    neg = (words < 0).astype(np.int64)
    nib = mag | (np.roll(neg, 1, axis=-1) << 3)   # nibble e gets the sign of code e-1
    nib = nib.reshape(c.shape)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: int8 codes [R, 2 * bytes]."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    if p.shape[-1] % 4:
        raise ValueError("packed row length must be a multiple of 4 bytes")
    nib = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int64)
    nib[..., 0::2] = p & 0xF
    nib[..., 1::2] = p >> 4
    words = nib.reshape(nib.shape[:-1] + (nib.shape[-1] // 8, 8))
    mag = words & 7
    neg = np.roll(words >> 3, -1, axis=-1)          # sign of code e sits in nibble e+1
    codes = np.where(neg == 1, -mag, mag)
    return codes.reshape(nib.shape).astype(np.int8)


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

def quantize_act(X: np.ndarray, spec: dict, mode: str = "group128", g: int = GROUP):
    """Oracle of quantize_act: transform, then per-group or RRS per-token INT4.

    ``g`` is the quantization group ([Paro] section 2.3 uses 128; other
    group sizes are a knob of the same quantizer).  Returns dict(qa=packed
    uint8 [M, K/2], sa=float64 [M, K/g], codes, ratio, xt=transformed
    activations, s=RRS group scales or None).
    """
    xt = transform_act(X, spec)
    if mode == "group128":
        codes, sa, ratio = quantize_groups(xt, g)
        s = None
    elif mode == "rrs":
        codes, sa, s, ratio = quantize_rrs(xt, g)
    else:
        raise ValueError(mode)
    return {"qa": pack_int4(codes), "sa": sa, "codes": codes, "ratio": ratio, "xt": xt, "s": s}


def pack_weight(W: np.ndarray, spec: dict, g: int = GROUP):
    """Oracle of pack_weight: W_tilde = T_w W, per-(output channel, group) INT4.

    W is [K, N].  Returns dict(qw=packed uint8 [N, K/2], sw=float64 [N, K/g],
    codes [N, K], ratio [N, K], wt=W_tilde [K, N]).
    """
    wt = transform_weight(W, spec)
    codes, sw, ratio = quantize_groups(wt.T, g)
    return {"qw": pack_int4(codes), "sw": sw, "codes": codes, "ratio": ratio, "wt": wt}


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
