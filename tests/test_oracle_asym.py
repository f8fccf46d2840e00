"""Pins of the oracle's asymmetric (s, z) quantizer and its GEMM.

The pages give the idea, not a worked example: [Paro] (the independent
rotation article) section 2.3 lets each 128-channel group share (s, z); the
Rotated Runtime Smooth page's symbol table writes q = round(x * scale) +
offset.  The oracle reads this as min/max round-to-nearest with zero kept in
the range.  These tests tie that reading to closed forms worked out by hand,
to the plain unsigned uniform quantizer it reduces to, to its error bound,
and the GEMM to a brute-force product of dequantized values (a different
formula from the oracle's centred integer accumulators).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_closed_form_linear_ramp():
    # 128 points from -1 to 2: lo = -1, hi = 2, s = 3 / 15 = 0.2, z = rne(1 / 0.2) = 5;
    # code k = rne(x_k / 0.2) + 5 = rne(15 k / 127)
    x = np.linspace(-1.0, 2.0, 128)[None, :]
    codes, s, z, ratio, zratio = oracle.quantize_groups_asym(x)
    assert s[0, 0] == pytest.approx(0.2, rel=1e-15)
    assert z[0, 0] == 5
    k = np.arange(128)
    np.testing.assert_array_equal(codes[0], np.rint(15.0 * k / 127.0).astype(np.uint8))
    assert codes[0, 0] == 0 and codes[0, -1] == 15


def test_golden_group():
    """A hand-worked group (tests/golden/asym_group_example.json)."""
    with open(os.path.join(GOLDEN, "asym_group_example.json")) as fh:
        ex = json.load(fh)
    x = np.zeros((1, 128))
    x[0, :len(ex["x"])] = ex["x"]
    codes, s, z, _, _ = oracle.quantize_groups_asym(x)
    assert s[0, 0] == pytest.approx(ex["s"], rel=1e-15)
    assert z[0, 0] == ex["z"]
    np.testing.assert_array_equal(codes[0, :len(ex["x"])], ex["codes"])
    np.testing.assert_array_equal(codes[0, len(ex["x"]):], ex["z"])  # the zero channels
    assert oracle.pack_uint4(codes)[0, :len(ex["packed_bytes"])].tolist() == ex["packed_bytes"]


def test_nonnegative_group_is_the_unsigned_uniform_quantizer():
    rng = np.random.default_rng(1)
    x = rng.exponential(1.0, size=(5, 256))
    codes, s, z, _, _ = oracle.quantize_groups_asym(x)
    assert np.all(z == 0)
    step = x.reshape(5, 2, 128).max(axis=2) / 15.0
    np.testing.assert_allclose(s, step, rtol=1e-15)
    expect = np.rint(x / np.repeat(step, 128, axis=1))
    np.testing.assert_array_equal(codes, expect.astype(np.uint8))


def test_nonpositive_group_uses_zero_point_15():
    rng = np.random.default_rng(2)
    x = -rng.exponential(1.0, size=(3, 128))
    codes, s, z, _, _ = oracle.quantize_groups_asym(x)
    assert np.all(z == 15)
    np.testing.assert_allclose(s[:, 0], -x.min(axis=1) / 15.0, rtol=1e-15)
    assert np.all(codes[np.arange(3), x.argmin(axis=1)] == 0)


def test_zero_group_and_zero_is_exact():
    x = np.zeros((2, 256))
    x[1, 128:] = np.linspace(-3.0, 5.0, 128)
    codes, s, z, _, _ = oracle.quantize_groups_asym(x)
    assert s[0, 0] == 0 and z[0, 0] == 0 and not codes[0].any()
    xh = oracle.dequantize_asym(codes, s, z)
    assert not xh[0].any()
    # zero inside a live group dequantizes to exactly zero (code == z)
    xz = np.array([[0.0, 1.0, -0.37] + [0.25] * 125])
    c2, s2, z2, _, _ = oracle.quantize_groups_asym(xz)
    assert oracle.dequantize_asym(c2, s2, z2)[0, 0] == 0.0


def test_range_and_error_bound():
    """codes and zero points in [0, 15]; |x - x_hat| <= s / 2 (round to nearest)."""
    rng = np.random.default_rng(3)
    xs = [rng.standard_normal((8, 512)), rng.standard_normal((8, 512)) + 3.0,
          rng.exponential(2.0, (8, 512)) - 0.1, rng.standard_t(2, (8, 512))]
    for x in xs:
        codes, s, z, _, _ = oracle.quantize_groups_asym(x)
        assert codes.max() <= 15 and z.min() >= 0 and z.max() <= 15
        err = np.abs(x - oracle.dequantize_asym(codes, s, z))
        assert np.all(err <= np.repeat(s, 128, axis=1) * (0.5 + 1e-12))


def test_asymmetric_beats_symmetric_on_one_sided_data():
    """16 levels over [0, max] against 8 over [0, max]: the asymmetric error is smaller."""
    rng = np.random.default_rng(4)
    x = rng.exponential(1.0, size=(16, 1024))
    ca, sa_, za, _, _ = oracle.quantize_groups_asym(x)
    cs, ss, _ = oracle.quantize_groups(x)
    ea = np.abs(x - oracle.dequantize_asym(ca, sa_, za)).mean()
    es = np.abs(x - oracle.dequantize(cs, ss)).mean()
    assert ea < 0.6 * es


def test_pack_uint4_layout_and_round_trip():
    # word 0 of a 32-code chunk (pair (0, 3), word 3 zero): unsigned fields f_k = u
    # in X = sum_k f_k << 6k; 1 -> X 0; 2 -> 7; 15 -> 12-15; 7 -> 24-26; 8 -> 33;
    # 9 -> 36, 39; 10 -> 43, 45.  X[32:64] bit q (= X - 32) goes to word 0 when
    # q mod 6 is 4 or 5 (q = 4, 11), to word 3 when it is 0 or 1 (q = 1, 7, 13)
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, :8] = [1, 2, 15, 0, 7, 8, 9, 10]
    assert oracle.pack_uint4(codes).tolist() == [[0x91, 0xF8, 0x00, 0x07] + [0] * 8 + [0x82, 0x20, 0x00, 0x00]]
    rng = np.random.default_rng(5)
    c = rng.integers(0, 16, size=(4, 256)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.unpack_uint4(oracle.pack_uint4(c)), c)
    with pytest.raises(ValueError):
        oracle.pack_uint4(np.array([[16] + [0] * 31]))


def test_weight_code_sums_brute_force():
    rng = np.random.default_rng(6)
    codes = rng.integers(-7, 8, size=(5, 384)).astype(np.int8)
    packed = oracle.pack_int4(codes)
    cw = oracle.weight_code_sums(packed)
    for n in range(5):
        for gi in range(3):
            assert cw[n, gi] == int(codes[n, gi * 128:(gi + 1) * 128].astype(np.int64).sum())


def test_asym_gemm_equals_dequantized_product():
    """Y from centred integer accumulators equals x_hat w_hat^T from the dequantized
    operands (float64 rounding only), at two group counts and a ragged N."""
    rng = np.random.default_rng(7)
    for M, K, N in ((3, 128, 5), (7, 512, 33)):
        x = rng.standard_normal((M, K)) + rng.uniform(-1, 2, size=(M, 1))
        w = rng.standard_normal((N, K)) * 0.02
        ca, sa, za, _, _ = oracle.quantize_groups_asym(x)
        cw, sw, _ = oracle.quantize_groups(w)
        y = oracle.w4a4_gemm_asym(oracle.pack_uint4(ca), sa, za, oracle.pack_int4(cw), sw, "f64")
        xh = oracle.dequantize_asym(ca, sa, za)
        wh = oracle.dequantize(cw, sw)
        ref = xh @ wh.T
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_quantize_act_asym_mode():
    rng = np.random.default_rng(8)
    X = rng.standard_normal((4, 256)) + 0.5
    spec = {"kind": "hadamard", "block": 128, "signs": None}
    a = oracle.quantize_act(X, spec, "group128_asym")
    xt = oracle.transform_act(X, spec)
    codes, s, z, _, _ = oracle.quantize_groups_asym(xt)
    np.testing.assert_array_equal(oracle.unpack_uint4(a["qa"]), codes)
    np.testing.assert_array_equal(a["za"], z)
    np.testing.assert_allclose(a["sa"], s, rtol=0)
