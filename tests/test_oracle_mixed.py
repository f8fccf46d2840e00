"""Pins of the oracle's 8-bit groups for extreme outliers.

[Paro] (the independent rotation article) section 4.1 lists mixed precision,
an 8-bit representation for extreme outliers, among the remedies for
outlier-heavy layers, beside more rotation layers and smaller groups.  The
oracle reads it as caller-named 128-channel groups quantized symmetrically
with 225 levels (q8 in [-112, 112]), split exactly into two INT4 planes
(q8 = 15 h + l) so that the INT4 GEMM computes them against a weight
matrix with those groups appended again.  These tests pin the split by
brute force, the quantizer against its closed form and error bound, and the
two-plane GEMM against the plain one-code definition and a dequantized
product.
"""
import numpy as np

import oracle


def test_split_covers_every_8bit_code():
    q8 = np.arange(-oracle.Q8MAX, oracle.Q8MAX + 1)
    h, lo = oracle.split_q8(q8)
    assert h.min() >= -7 and h.max() <= 7 and lo.min() >= -7 and lo.max() <= 7
    np.testing.assert_array_equal(15 * h + lo, q8)
    # the pair is unique: no other (h, l) in [-7, 7]^2 gives the same value
    hs, ls = np.meshgrid(np.arange(-7, 8), np.arange(-7, 8), indexing="ij")
    vals = (15 * hs + ls).ravel()
    assert len(np.unique(vals)) == 225 and vals.min() == -112 and vals.max() == 112


def test_8bit_group_closed_form_and_bound():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 384))
    x[:, 130] = 40.0                        # an extreme outlier channel in group 1
    q, sc, ratio = oracle.quantize_groups_mixed(x, [1])
    c4, s4, _ = oracle.quantize_groups(x)
    np.testing.assert_array_equal(q[:, :128], c4[:, :128])       # 4-bit groups unchanged
    np.testing.assert_array_equal(q[:, 256:], c4[:, 256:])
    m = np.abs(x[:, 128:256]).max(axis=1)
    np.testing.assert_allclose(sc[:, 1], m / 112.0, rtol=1e-15)
    np.testing.assert_array_equal(q[:, 128:256], np.rint(x[:, 128:256] / (m / 112.0)[:, None]))
    assert np.all(np.abs(q[:, 130]) == 112)
    xh = q[:, 128:256] * sc[:, 1][:, None]
    assert np.all(np.abs(xh - x[:, 128:256]) <= sc[:, 1][:, None] * (0.5 + 1e-12))
    # the other channels of the outlier group: a 16 times finer step than at 4 bits
    # (at 4 bits almost all of them round to 0)
    e8 = np.abs(xh - x[:, 128:256])[:, np.arange(128) != 2].mean()
    e4 = np.abs(c4[:, 128:256] * s4[:, 1][:, None] - x[:, 128:256])[:, np.arange(128) != 2].mean()
    assert e8 < e4 / 4


def test_two_plane_gemm_equals_the_one_code_definition():
    rng = np.random.default_rng(12)
    M, K, N = 5, 512, 23
    spec = {"kind": "hadamard", "block": 128, "signs": None}
    X = rng.standard_normal((M, K))
    X[:, 300] *= 300.0
    W = rng.standard_normal((K, N)) * 0.02
    groups8 = [2, 0]
    a = oracle.quantize_act(X, spec, "group128_mixed", order=groups8)
    w = oracle.pack_weight(W, spec)
    cw_ext, sw_ext = oracle.extend_weight_groups(w["codes"], w["sw"], groups8)
    assert cw_ext.shape == (N, K + 256) and sw_ext.shape == (N, 6)
    # what the library computes: the plain INT4 GEMM over the extended K
    y_planes = oracle.w4a4_gemm(a["qa"], a["sa"], oracle.pack_int4(cw_ext), sw_ext, "f64")
    # the definition: one code per channel (q8 in the 8-bit groups)
    y_def = oracle.mixed_gemm_reference(a["codes"], a["scales"], groups8, w["codes"], w["sw"])
    np.testing.assert_allclose(y_planes, y_def, rtol=1e-12, atol=1e-12 * np.abs(y_def).max())
    # and a brute-force product of the dequantized operands
    xh = a["codes"] * np.repeat(a["scales"], 128, axis=1)
    wh = oracle.dequantize(w["codes"], w["sw"])
    np.testing.assert_allclose(y_def, xh @ wh.T, rtol=1e-12, atol=1e-12 * np.abs(y_def).max())
    # planes: h in place, l appended, scales 15 s8 and s8
    planes = oracle.unpack_int4(a["qa"]).astype(np.int64)
    for j, gi in enumerate(groups8):
        h, lo = oracle.split_q8(a["codes"][:, gi * 128:(gi + 1) * 128])
        np.testing.assert_array_equal(planes[:, gi * 128:(gi + 1) * 128], h)
        np.testing.assert_array_equal(planes[:, K + j * 128:K + (j + 1) * 128], lo)
        np.testing.assert_allclose(a["sa"][:, gi], 15.0 * a["scales"][:, gi], rtol=1e-15)
        np.testing.assert_allclose(a["sa"][:, 4 + j], a["scales"][:, gi], rtol=0)


def test_mixed_with_no_groups_is_the_4bit_quantizer():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((3, 256))
    spec = {"kind": "hadamard", "block": 128, "signs": None}
    a = oracle.quantize_act(X, spec, "group128_mixed", order=[])
    b = oracle.quantize_act(X, spec, "group128")
    np.testing.assert_array_equal(a["qa"], b["qa"])
    np.testing.assert_array_equal(a["sa"], b["sa"])
